"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Small sizes (the oracle finishes in seconds) that still span several 16-row
slabs, several 16-column tiles, ragged staging chunks and ragged checkpoint
intervals, on the recipes of all five workloads, in both state precisions.

Tolerances.  Over these short horizons the recurrence does not amplify
rounding noticeably, so the fp32 path is held to 2e-5 max-abs on y, H_T and
checkpoints (tighter than the stated 1e-4 / 2e-2: the per-step fp32 error is
~1e-7 and grows by far less than 100x within ~100 steps), and the fp64 path to
1e-11.  Gradients are compared per tensor as max|g - g_ref| <= tau *
max(1, max|g_ref|), tau = 1e-4 (fp32) / 1e-10 (fp64).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from m2rnn_inputs import WORKLOADS, WORKLOAD_ORDER, Workload, make_inputs, to_device
from matrix_state_nonlinear_amd import m2rnn_bwd, m2rnn_fwd, m2rnn_gates, m2rnn_workspace_bytes

pytestmark = pytest.mark.gpu

TOL_Y = {"float32": 2e-5, "float64": 1e-11}
TAU_G = {"float32": 1e-4, "float64": 1e-10}


def np_(t):
    return None if t is None else t.detach().cpu().numpy().astype(np.float64)


def gpu_forward(inp, sd, C=0):
    d = to_device(inp, sd)
    f = m2rnn_gates(d["logit"], inp.wl.gate, d["alpha"], d["beta"])
    y, HT, ckpt = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], C)
    torch.cuda.synchronize()
    return d, f, y, HT, ckpt


def oracle_forward(inp, C=0, keep=False):
    f = oracle.gates(inp.wl.gate, inp.logit, inp.alpha, inp.beta)
    return f, oracle.forward(inp.k, inp.v, inp.q, f, inp.W, inp.w_r, inp.H0, C=C,
                             keep_states=keep)


def small(name, **kw):
    wl = WORKLOADS[name]
    base = dict(B=min(wl.B, 2), T=77, N=min(wl.N, 2))
    base.update(kw)
    return wl.replace(**base)


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


# ---------------------------------------------------------------- gates

@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("name", ["tiny_fp32", "long_t16k_k64"])
def test_gates(name, sd):
    wl = small(name, T=300)
    inp = make_inputs(wl)
    inp.logit[0, :6, 0] = [-200.0, -30.0, -1e-3, 0.0, 30.0, 200.0]
    d = to_device(inp, sd)
    f = np_(m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"]))
    ref = oracle.gates(wl.gate, inp.logit.astype(np.float64 if sd == "float64" else np.float32),
                       inp.alpha, inp.beta)
    tol = 2e-7 if sd == "float32" else 1e-15
    assert maxerr(f, ref) <= tol
    assert np.all((f >= 0) & (f <= 1))


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_forward_workload_recipes(name, sd):
    wl = small(name)
    inp = make_inputs(wl)
    C = 16
    _, f, y, HT, ckpt = gpu_forward(inp, sd, C=C)
    fo, o = oracle_forward(inp, C=C)
    tol = TOL_Y[sd]
    ey, eh, ec = maxerr(np_(y), o["y"]), maxerr(np_(HT), o["HT"]), maxerr(np_(ckpt), o["ckpt"])
    print(f"{name} {sd}: y {ey:.2e} HT {eh:.2e} ckpt {ec:.2e}")
    assert ey <= tol and eh <= tol and ec <= tol


SHAPES = [  # (K, V): slab and tile edge cases
    (1, 1), (15, 5), (16, 16), (17, 17), (40, 40), (33, 72), (24, 100), (256, 16), (48, 128),
]


@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("K,V", SHAPES)
def test_forward_shapes_with_h0_and_ragged_checkpoints(K, V, sd):
    wl = WORKLOADS["fp32_k64"].replace(B=2, T=45, N=3, K=K, V=V, kq_scale=1 / math.sqrt(K),
                                       v_scale=1 / math.sqrt(V), w_scale=1 / math.sqrt(V))
    inp = make_inputs(wl, with_h0=True)
    C = 7
    _, f, y, HT, ckpt = gpu_forward(inp, sd, C=C)
    fo, o = oracle_forward(inp, C=C)
    tol = TOL_Y[sd]
    assert maxerr(np_(y), o["y"]) <= tol
    assert maxerr(np_(HT), o["HT"]) <= tol
    assert maxerr(np_(ckpt), o["ckpt"]) <= tol


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 200])
def test_forward_sequence_lengths(T):
    wl = small("long_t16k_k64", T=T, B=1)
    inp = make_inputs(wl)
    _, f, y, HT, ckpt = gpu_forward(inp, "float32", C=32)
    fo, o = oracle_forward(inp, C=32)
    assert maxerr(np_(y), o["y"]) <= TOL_Y["float32"]
    assert maxerr(np_(HT), o["HT"]) <= TOL_Y["float32"]


def test_forward_gate_one_keeps_state_exactly():
    wl = small("fp32_k64", T=40)
    inp = make_inputs(wl, with_h0=True)
    d = to_device(inp, "float32")
    f = torch.ones_like(d["logit"])
    y, HT, _ = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"])
    assert torch.equal(HT, d["H0"])
    o = oracle.forward(inp.k, inp.v, inp.q, np.ones_like(inp.logit), inp.W, inp.w_r, inp.H0)
    assert maxerr(np_(y), o["y"]) <= 1e-6


def test_forward_gate_zero_w_zero_is_tanh_outer():
    wl = small("fp32_k64", T=5)
    inp = make_inputs(wl)
    d = to_device(inp, "float32")
    f = torch.zeros_like(d["logit"])
    W = torch.zeros_like(d["W"])
    _, HT, _ = m2rnn_fwd(d["k"], d["v"], d["q"], f, W, d["w_r"])
    want = np.tanh(inp.k[:, -1, :, :, None].astype(np.float64) * inp.v[:, -1, :, None, :])
    assert maxerr(np_(HT), want) <= 3e-7


def test_forward_chunked_equals_full_bitwise_and_deterministic():
    wl = small("long_t16k_k64", T=150, B=2)
    inp = make_inputs(wl)
    d = to_device(inp, "float32")
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
    y, HT, _ = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"])
    y2, HT2, _ = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"])
    assert torch.equal(y, y2) and torch.equal(HT, HT2)
    T1 = 61
    sl = lambda t, a, b: t[:, a:b].contiguous()  # noqa: E731
    ya, Ha, _ = m2rnn_fwd(sl(d["k"], 0, T1), sl(d["v"], 0, T1), sl(d["q"], 0, T1),
                          sl(f, 0, T1), d["W"], d["w_r"])
    yb, Hb, _ = m2rnn_fwd(sl(d["k"], T1, 150), sl(d["v"], T1, 150), sl(d["q"], T1, 150),
                          sl(f, T1, 150), d["W"], d["w_r"], Ha)
    assert torch.equal(torch.cat([ya, yb], 1), y)
    assert torch.equal(Hb, HT)


def test_forward_state_stays_in_unit_box():
    wl = small("long_t16k_k64", T=500, B=2, N=4)
    inp = make_inputs(wl)
    _, f, y, HT, ckpt = gpu_forward(inp, "float32", C=1)
    assert float(ckpt.abs().max()) <= 1.0


# ---------------------------------------------------------------- backward

def gpu_backward(inp, sd, C):
    d, f, y, HT, ckpt = gpu_forward(inp, sd, C=C)
    g = m2rnn_bwd(d["k"], d["v"], d["q"], inp.wl.gate, d["logit"], d["alpha"], d["beta"], f,
                  d["W"], d["w_r"], d["H0"], ckpt, C, d["dy"], d["dHT"])
    torch.cuda.synchronize()
    return {k_: np_(v_) for k_, v_ in g.items()}


def oracle_backward(inp):
    f = oracle.gates(inp.wl.gate, inp.logit, inp.alpha, inp.beta)
    return oracle.backward(inp.k, inp.v, inp.q, f, inp.W, inp.w_r, inp.dy, inp.H0, inp.dHT,
                           gate_kind=inp.wl.gate, logit=inp.logit, alpha=inp.alpha,
                           beta=inp.beta)


def check_grads(g, ref, tau, label=""):
    worst = {}
    for name, r in ref.items():
        if name == "df" or r is None:
            continue
        scale = max(1.0, float(np.max(np.abs(r))))
        err = maxerr(g[name], r) / scale
        worst[name] = err
    print(label, {k_: f"{v_:.1e}" for k_, v_ in worst.items()})
    bad = {k_: v_ for k_, v_ in worst.items() if not v_ <= tau}
    assert not bad, bad


@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_backward_workload_recipes(name, sd):
    wl = small(name, T=70)
    inp = make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)
    g = gpu_backward(inp, sd, C=16)
    check_grads(g, oracle_backward(inp), TAU_G[sd], f"{name} {sd}")


@pytest.mark.parametrize("K,V,C", [(1, 1, 1), (17, 40, 7), (40, 72, 64), (33, 100, 5),
                                   (16, 128, 3), (20, 20, 3), (32, 32, 4), (9, 24, 2),
                                   (9, 10, 3), (70, 12, 4)])
def test_backward_shapes(K, V, C):
    # V = 20, 24, 32: the column sums of dw_r, dalpha, dbeta read 3 or 2 rows
    # per load (V in 17..32), V <= 16: 4 rows, V >= 64: one.  V = 10, 12: one
    # value tile with padding columns (the reverse role's dv with 4-byte stores),
    # K = 9 one slab with padding rows, K = 70 five slabs (the dv partials summed)
    wl = WORKLOADS["fwd_bwd_k32_v128"].replace(B=2, T=29, N=2, K=K, V=V,
                                               kq_scale=1 / math.sqrt(K),
                                               v_scale=1 / math.sqrt(V), w_scale=1 / math.sqrt(V))
    inp = make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)
    for sd in ("float32", "float64"):
        g = gpu_backward(inp, sd, C=C)
        check_grads(g, oracle_backward(inp), TAU_G[sd], f"K{K} V{V} C{C} {sd}")


def test_backward_deterministic():
    wl = small("fwd_bwd_k32_v128", T=50)
    inp = make_inputs(wl, with_dy=True)
    g1 = gpu_backward(inp, "float32", C=16)
    g2 = gpu_backward(inp, "float32", C=16)
    for k_ in g1:
        if g1[k_] is not None:
            assert np.array_equal(g1[k_], g2[k_]), k_


@pytest.mark.parametrize("sd", ["float32", "float64"])
def test_forward_checkpoints_every_c_steps_inside_chunks(sd):
    """Checkpoints are written after the step they follow, wherever it falls
    in the forward's unrolled staging chunk (8, 16 or 32 steps): every
    checkpoint must equal the state the per-step interval (C = 1) stores, bit
    for bit, and the oracle's state.  T = 157 leaves a ragged last chunk."""
    wl = small("long_t16k_k64", T=157, B=2)
    inp = make_inputs(wl)
    _, f, y1, HT1, ck1 = gpu_forward(inp, sd, C=1)
    fo, o = oracle_forward(inp, C=1)
    assert maxerr(np_(ck1), o["ckpt"]) <= TOL_Y[sd]
    for C in (2, 3, 4, 8, 16, 32, 33, 64):
        _, _, y, HT, ck = gpu_forward(inp, sd, C=C)
        assert torch.equal(y, y1) and torch.equal(HT, HT1), C
        assert torch.equal(ck, ck1[:, :, ::C].contiguous()), C


# ---------------------------------------------------------------- empty calls

@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("B,T,N", [(2, 0, 3), (0, 9, 3), (2, 9, 0)])
def test_empty_batch_sequence_or_heads(B, T, N, sd):
    """No steps or no rows: the oracle's results for zero tokens.  H_T is H_0
    and dH_0 is dH_T (copied bit for bit), dW, dw_r, dalpha and dbeta are zero,
    and the per-token outputs and checkpoints are empty."""
    wl = WORKLOADS["fwd_bwd_k32_v128"].replace(B=B, T=T, N=N, K=20, V=24)
    inp = make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)
    C = 4
    d, f, y, HT, ckpt = gpu_forward(inp, sd, C=C)
    _, o = oracle_forward(inp, C=C)
    assert tuple(y.shape) == o["y"].shape and tuple(ckpt.shape) == o["ckpt"].shape
    assert torch.equal(HT, d["H0"])
    g = m2rnn_bwd(d["k"], d["v"], d["q"], wl.gate, d["logit"], d["alpha"], d["beta"], f,
                  d["W"], d["w_r"], d["H0"], ckpt, C, d["dy"], d["dHT"])
    torch.cuda.synchronize()
    ref = oracle_backward(inp)
    assert torch.equal(g["dH0"], d["dHT"])
    for name, r in ref.items():
        if name == "df" or r is None:
            continue
        assert tuple(g[name].shape) == r.shape, name
        if r.size and name != "dH0":
            assert not np.any(r) and not torch.any(g[name]), name


# ---------------------------------------------------------------- stored rc

@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("K,V,C,NQ", [(64, 64, 4, 0), (17, 40, 7, 0), (33, 100, 5, 1),
                                      (16, 16, 4, 0), (48, 128, 2, 0), (64, 16, 8, 1)])
def test_stored_rc_forward_and_backward(K, V, C, NQ, sd):
    """The forward's optional rc output (rc_t = 1 / (1 + e^{2 A_t}) of every step)
    leaves y, H_T and the checkpoints bit for bit unchanged, matches the
    oracle's (1 - Z_t) / 2, and the backward given it returns exactly the
    results of the backward that recomputes the states (the states follow from
    rc by the interpolation alone, with the forward's arithmetic)."""
    wl = WORKLOADS["fwd_bwd_k32_v128"].replace(B=2, T=45, N=4 if NQ else 2, K=K, V=V, NQ=NQ,
                                               kq_scale=1 / math.sqrt(K),
                                               v_scale=1 / math.sqrt(V), w_scale=1 / math.sqrt(V))
    inp = make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)
    d = to_device(inp, sd)
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
    y0, HT0, ck0 = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], C)
    rc = torch.empty((wl.B, wl.N, wl.T, K, V), dtype=f.dtype, device=f.device)
    y1, HT1, ck1 = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], C, rc_out=rc)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(HT0, HT1) and torch.equal(ck0, ck1)
    fo, o = oracle_forward(inp, keep=True)
    rc_ref = np.transpose((1.0 - o["Z"]) / 2.0, (1, 2, 0, 3, 4))
    assert maxerr(np_(rc), rc_ref) <= TOL_Y[sd]
    args = (d["k"], d["v"], d["q"], wl.gate, d["logit"], d["alpha"], d["beta"], f, d["W"],
            d["w_r"], d["H0"], ck0, C, d["dy"], d["dHT"])
    g0 = m2rnn_bwd(*args)
    g1 = m2rnn_bwd(*args, rc=rc)
    torch.cuda.synchronize()
    for name in g0:
        if g0[name] is not None:
            assert torch.equal(g0[name], g1[name]), name


@pytest.mark.parametrize("K,V,T,C,NQ", [(32, 128, 45, 4, 0), (20, 120, 61, 6, 1), (48, 128, 130, 8, 0),
                                        (16, 113, 29, 64, 0), (64, 128, 200, 16, 2)])
def test_backward_interval_sweep_matches_the_oracle(K, V, T, C, NQ):
    """V > 112 (eight value tiles) with C a larger multiple of the backward's
    2-step chunk: the main kernel sweeps each checkpoint interval once (its
    states, and rc when recomputing, in a two-interval ring of the workspace)
    instead of a chunk-start pass.  Ragged K, V and T, shared q/k, an interval
    longer than T, both modes: the gradients match the oracle at the fp32
    tolerance and the two modes each other bit for bit."""
    N = 4 if NQ else 2
    wl = WORKLOADS["fwd_bwd_k32_v128"].replace(B=2, T=T, N=N, NQ=NQ, K=K, V=V,
                                               kq_scale=1 / math.sqrt(K),
                                               v_scale=1 / math.sqrt(V), w_scale=1 / math.sqrt(V))
    inp = make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)
    d = to_device(inp, "float32")
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
    rc = torch.empty((wl.B, wl.N, wl.T, K, V), dtype=f.dtype, device=f.device)
    _, _, ck = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], C, rc_out=rc)
    args = (d["k"], d["v"], d["q"], wl.gate, d["logit"], d["alpha"], d["beta"], f, d["W"],
            d["w_r"], d["H0"], ck, C, d["dy"], d["dHT"])
    g0 = m2rnn_bwd(*args)
    g1 = m2rnn_bwd(*args, rc=rc)
    torch.cuda.synchronize()
    for name in g0:
        if g0[name] is not None:
            assert torch.equal(g0[name], g1[name]), name
    check_grads({k_: np_(v_) for k_, v_ in g0.items() if v_ is not None}, oracle_backward(inp),
                TAU_G["float32"], f"sweep K{K} V{V} T{T} C{C} NQ{NQ}")


# ---------------------------------------------------------------- alignment

def _offset_view(shape, dtype, elems=1, dev="cuda:0"):
    """A contiguous tensor that starts `elems` elements into its storage, so it
    is aligned to its element type but not to 16 bytes."""
    n = int(np.prod(shape))
    return torch.empty(n + elems, dtype=dtype, device=dev)[elems:].view(shape)


@pytest.mark.parametrize("K,V,C", [(64, 64, 4), (32, 128, 6), (16, 16, 2), (40, 72, 3)])
def test_element_aligned_buffers_give_identical_results(K, V, C):
    """Arrays that are aligned to their element type but not to 16 bytes take
    the element-access paths of the kernels (the 16-byte ones need 16-byte
    addresses): results equal those with 16-byte aligned buffers, bit for bit.
    (The backward's workspace itself must be 16-byte aligned.)"""
    wl = WORKLOADS["fwd_bwd_k32_v128"].replace(B=2, T=37, N=2, K=K, V=V,
                                               kq_scale=1 / math.sqrt(K),
                                               v_scale=1 / math.sqrt(V), w_scale=1 / math.sqrt(V))
    inp = make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)
    d = to_device(inp, "float32")
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
    B, T, N = wl.B, wl.T, wl.N
    f32 = torch.float32
    rc0 = torch.empty((B, N, T, K, V), dtype=f32, device=f.device)
    y0, HT0, ck0 = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], C, rc_out=rc0)
    y1 = _offset_view((B, T, N, V), f32)
    HT1 = _offset_view((B, N, K, V), f32)
    ck1 = _offset_view((B, N, math.ceil(T / C), K, V), f32)
    rc1 = _offset_view((B, N, T, K, V), f32)
    nws = m2rnn_workspace_bytes(False, B, T, N, N, K, V, C, f32)
    ws1 = _offset_view((nws // 4 + 1,), f32)
    m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], C, out=(y1, HT1, ck1),
              rc_out=rc1, workspace=ws1.view(torch.uint8))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(HT0, HT1) and torch.equal(ck0, ck1)
    assert torch.equal(rc0, rc1)
    args = (d["k"], d["v"], d["q"], wl.gate, d["logit"], d["alpha"], d["beta"], f, d["W"],
            d["w_r"], d["H0"], ck0, C, d["dy"], d["dHT"])
    g0 = m2rnn_bwd(*args, rc=rc0)
    out = {"dv": _offset_view((B, T, N, V), f32), "dk": _offset_view((B, T, N, K), f32)}
    g1 = m2rnn_bwd(*args, rc=rc1, out=out)
    g2 = m2rnn_bwd(*args, rc=None, out=None)
    torch.cuda.synchronize()
    for name in g0:
        if g0[name] is not None:
            assert torch.equal(g0[name], g1[name]), name
            assert torch.equal(g0[name], g2[name]), name
