"""Pins of the float64 oracle against facts the pages and the mathematics fix.

None of these compares the oracle with itself: each checks a special case
with a closed form, a library routine (torch.nn.RNN, scipy), an identity,
brute force (finite differences) or an invariant of the recurrence.
Sources: review of "M²RNN: Non-Linear RNNs with Matrix-Valued States for
Scalable Language Modeling" (section 2.1 Eq. 10-12, section 2.2 Eq. 13/17,
section 2.5 Theorem 1, section 2.7 corrected backward) and the pararnn-torch
"ParaM2RNN" page ("Recurrence", "Jacobian class").
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from m2rnn_inputs import (GATE_EXP_SOFTPLUS, GATE_SIGMOID, WORKLOAD_ORDER,
                          WORKLOADS, make_inputs)


def _rand_case(seed, B=2, T=7, N=2, K=3, V=4, f_lo=0.05, f_hi=0.95, h0=True):
    rng = np.random.default_rng(seed)
    c = dict(
        k=rng.standard_normal((B, T, N, K)) * 0.7,
        v=rng.standard_normal((B, T, N, V)) * 0.7,
        q=rng.standard_normal((B, T, N, K)),
        f=rng.uniform(f_lo, f_hi, (B, T, N)),
        W=np.eye(V)[None] * 0.8 + rng.standard_normal((N, V, V)) * 0.3,
        w_r=rng.standard_normal((N, V)) * 0.5,
        H0=rng.uniform(-0.6, 0.6, (B, N, K, V)) if h0 else None,
    )
    return c


# ---------------------------------------------------------------- gates

def test_gate_sigmoid_matches_scipy():
    x = np.concatenate([np.linspace(-50, 50, 1001), [-1e3, 1e3, 0.0]])
    np.testing.assert_allclose(oracle.gates(GATE_SIGMOID, x), scipy.special.expit(x),
                               rtol=1e-15, atol=0)


def test_softplus_matches_logaddexp_and_is_finite():
    x = np.concatenate([np.linspace(-60, 60, 1201), [-1e4, 1e4]])
    sp = oracle.softplus(x)
    assert np.all(np.isfinite(sp))
    np.testing.assert_allclose(sp, np.logaddexp(0.0, x), rtol=1e-14, atol=1e-300)


def test_exp_softplus_alpha_one_is_sigmoid_of_minus():
    # review section 2.2: with alpha = 1 the gate equals sigmoid(-a - beta)
    rng = np.random.default_rng(3)
    a = rng.standard_normal((4, 9, 5)) * 4
    beta = rng.uniform(-2, 2, 5)
    f = oracle.gates(GATE_EXP_SOFTPLUS, a, np.ones(5), beta)
    np.testing.assert_allclose(f, scipy.special.expit(-a - beta), rtol=1e-13, atol=0)


def test_exp_softplus_power_form():
    # Eq. 13: f = (1 + e^{a + beta})^{-alpha}, evaluated directly where it is safe
    rng = np.random.default_rng(4)
    a = rng.standard_normal((3, 6, 4))
    alpha = np.exp(rng.uniform(math.log(0.1), math.log(2.0), 4))
    beta = rng.uniform(-2, 2, 4)
    f = oracle.gates(GATE_EXP_SOFTPLUS, a, alpha, beta)
    np.testing.assert_allclose(f, (1.0 + np.exp(a + beta)) ** (-alpha), rtol=1e-13)
    assert np.all((f >= 0) & (f <= 1))


# ---------------------------------------------------------------- forward special cases

def test_f_one_keeps_state():
    # review section 2.1: f_t = 1 keeps the state, so H_t = H_0 for every t and the
    # readout is H_0^T q_t + w_r * v_t.
    c = _rand_case(1, T=9)
    f = np.ones_like(c["f"])
    o = oracle.forward(c["k"], c["v"], c["q"], f, c["W"], c["w_r"], c["H0"],
                       keep_states=True)
    for t in range(9 + 1):
        assert np.array_equal(o["H"][t], c["H0"])
    B, T, N, K = c["k"].shape
    for b in range(B):
        for t in range(T):
            for n in range(N):
                want = c["H0"][b, n].T @ c["q"][b, t, n] + c["w_r"][n] * c["v"][b, t, n]
                np.testing.assert_allclose(o["y"][b, t, n], want, rtol=1e-14, atol=1e-15)


def test_f_zero_w_zero_is_tanh_outer():
    # review section 2.1: f = 0 and W = 0 leave H_t = tanh(k_t v_t^T)
    c = _rand_case(2, T=6)
    f = np.zeros_like(c["f"])
    W = np.zeros_like(c["W"])
    o = oracle.forward(c["k"], c["v"], c["q"], f, W, c["w_r"], c["H0"], keep_states=True)
    B, T, N, K = c["k"].shape
    for b in range(B):
        for t in range(T):
            for n in range(N):
                want = np.tanh(np.outer(c["k"][b, t, n], c["v"][b, t, n]))
                np.testing.assert_array_equal(o["H"][t + 1][b, n], want)


def test_w_zero_closed_form():
    # With W = 0, Eq. (11) is a linear recurrence in H with input (1-f_t) tanh(k_t v_t^T):
    # H_T = (prod_s f_s) H_0 + sum_s (1 - f_s) (prod_{r > s} f_r) tanh(k_s v_s^T).
    c = _rand_case(3, T=11, B=3, N=2, K=4, V=5)
    W = np.zeros_like(c["W"])
    o = oracle.forward(c["k"], c["v"], c["q"], c["f"], W, c["w_r"], c["H0"])
    f = c["f"]
    T = f.shape[1]
    # reverse cumulative products prod_{r > s} f_r, computed through log-free cumprod
    tail = np.ones_like(f)
    for s in range(T - 2, -1, -1):
        tail[:, s] = tail[:, s + 1] * f[:, s + 1]
    total = tail[:, 0] * f[:, 0]
    want = total[:, :, None, None] * c["H0"]
    for s in range(T):
        ks = c["k"][:, s]
        vs = c["v"][:, s]
        want = want + ((1 - f[:, s]) * tail[:, s])[:, :, None, None] * np.tanh(
            ks[..., :, None] * vs[..., None, :])
    np.testing.assert_allclose(o["HT"], want, rtol=1e-13, atol=1e-14)


def test_theorem1_matches_torch_rnn_forward_and_backward():
    # review section 2.5 / Theorem 1: f = 0, w_r = 0, q = k = e_1 embeds the tanh RNN
    # h_t = tanh(W^T h_{t-1} + v_t) in row 1; y_t = h_t, the other rows stay zero.
    rng = np.random.default_rng(5)
    B, T, N, K, V = 3, 17, 1, 4, 6
    v = rng.standard_normal((B, T, N, V))
    W = rng.standard_normal((N, V, V)) * 0.6
    e1 = np.zeros(K)
    e1[0] = 1.0
    k = np.broadcast_to(e1, (B, T, N, K)).copy()
    q = k.copy()
    f = np.zeros((B, T, N))
    w_r = np.zeros((N, V))
    o = oracle.forward(k, v, q, f, W, w_r, keep_states=True)
    assert np.all(o["H"][:, :, :, 1:, :] == 0.0)

    rnn = torch.nn.RNN(V, V, nonlinearity="tanh", bias=False, batch_first=True).double()
    with torch.no_grad():
        rnn.weight_ih_l0.copy_(torch.eye(V, dtype=torch.float64))
        rnn.weight_hh_l0.copy_(torch.from_numpy(W[0].T.copy()))
    x = torch.from_numpy(v[:, :, 0, :].copy()).requires_grad_(True)
    h, _ = rnn(x)
    np.testing.assert_allclose(o["y"][:, :, 0, :], h.detach().numpy(), rtol=1e-12, atol=1e-13)

    dy = rng.standard_normal((B, T, N, V))
    (h * torch.from_numpy(dy[:, :, 0, :].copy())).sum().backward()
    g = oracle.backward(k, v, q, f, W, w_r, dy)
    np.testing.assert_allclose(g["dv"][:, :, 0, :], x.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dW"][0], rnn.weight_hh_l0.grad.numpy().T, rtol=1e-11,
                               atol=1e-12)


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_state_stays_in_unit_box(name):
    # review section 2.1: H_0 = 0 and f in [0, 1] keep every entry in [-1, 1]
    wl = WORKLOADS[name]
    wl = wl.replace(B=1, T=min(wl.T, 96), N=min(wl.N, 4))
    inp = make_inputs(wl)
    f = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    assert np.all((f >= 0) & (f <= 1))
    o = oracle.forward(inp.k, inp.v, inp.q, f, inp.W, inp.w_r, keep_states=True)
    assert np.abs(o["H"]).max() <= 1.0
    assert np.abs(o["Z"]).max() <= 1.0


def test_row_independence():
    # W mixes value columns only, so each key row is its own recurrence; the readout
    # sums the rows (review section 1.2 / 2.5).
    c = _rand_case(6, T=8, K=5, V=4)
    full = oracle.forward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], c["H0"])
    acc = np.zeros_like(full["y"])
    zero_wr = np.zeros_like(c["w_r"])
    for i in range(5):
        sl = slice(i, i + 1)
        o = oracle.forward(c["k"][..., sl], c["v"], c["q"][..., sl], c["f"], c["W"], zero_wr,
                           c["H0"][:, :, sl, :])
        acc += o["y"]
        np.testing.assert_allclose(o["HT"][:, :, 0], full["HT"][:, :, i], rtol=0, atol=1e-15)
    acc += c["w_r"][None, None] * c["v"]
    np.testing.assert_allclose(acc, full["y"], rtol=1e-13, atol=1e-14)
    perm = np.array([3, 0, 4, 2, 1])
    p = oracle.forward(c["k"][..., perm], c["v"], c["q"][..., perm], c["f"], c["W"], c["w_r"],
                       c["H0"][:, :, perm, :])
    np.testing.assert_allclose(p["y"], full["y"], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(p["HT"], full["HT"][:, :, perm, :])


def test_chunked_equals_full():
    c = _rand_case(7, T=13)
    full = oracle.forward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], c["H0"], C=4)
    T1 = 5
    a = oracle.forward(c["k"][:, :T1], c["v"][:, :T1], c["q"][:, :T1], c["f"][:, :T1], c["W"],
                       c["w_r"], c["H0"])
    b = oracle.forward(c["k"][:, T1:], c["v"][:, T1:], c["q"][:, T1:], c["f"][:, T1:], c["W"],
                       c["w_r"], a["HT"])
    np.testing.assert_array_equal(np.concatenate([a["y"], b["y"]], axis=1), full["y"])
    np.testing.assert_array_equal(b["HT"], full["HT"])
    # ckpt[c] = H_{cC}: it is the state a run of length cC ends in
    for cidx in range(full["ckpt"].shape[2]):
        t = cidx * 4
        if t == 0:
            np.testing.assert_array_equal(full["ckpt"][:, :, 0], c["H0"])
            continue
        o = oracle.forward(c["k"][:, :t], c["v"][:, :t], c["q"][:, :t], c["f"][:, :t], c["W"],
                           c["w_r"], c["H0"])
        np.testing.assert_array_equal(full["ckpt"][:, :, cidx], o["HT"])


def test_causality():
    c = _rand_case(8, T=12)
    base = oracle.forward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], c["H0"])
    t0 = 6
    rng = np.random.default_rng(9)
    c2 = {k_: (v_.copy() if isinstance(v_, np.ndarray) else v_) for k_, v_ in c.items()}
    for key in ("k", "v", "q"):
        c2[key][:, t0 + 1:] += rng.standard_normal(c2[key][:, t0 + 1:].shape)
    c2["f"][:, t0 + 1:] = rng.uniform(0, 1, c2["f"][:, t0 + 1:].shape)
    pert = oracle.forward(c2["k"], c2["v"], c2["q"], c2["f"], c["W"], c["w_r"], c["H0"])
    np.testing.assert_array_equal(pert["y"][:, :t0 + 1], base["y"][:, :t0 + 1])
    assert not np.allclose(pert["y"][:, t0 + 1:], base["y"][:, t0 + 1:])


# ---------------------------------------------------------------- Jacobian and backward

def _one_step(Hp, k, v, f, W):
    return f * Hp + (1 - f) * np.tanh(Hp @ W + np.outer(k, v))


def test_dense_jacobian_matches_finite_differences():
    rng = np.random.default_rng(10)
    for K, V in [(2, 3), (3, 3), (4, 2)]:
        Hp = rng.uniform(-0.8, 0.8, (K, V))
        k = rng.standard_normal(K)
        v = rng.standard_normal(V)
        W = rng.standard_normal((V, V)) * 0.7
        f = 0.37
        Z = np.tanh(Hp @ W + np.outer(k, v))
        J = oracle.step_jacobian_dense(Hp, Z, f, W)
        h = 1e-6
        Jfd = np.empty((K * V, K * V))
        for idx in range(K * V):
            e = np.zeros(K * V)
            e[idx] = h
            Jfd[:, idx] = ((_one_step(Hp + e.reshape(K, V), k, v, f, W)
                            - _one_step(Hp - e.reshape(K, V), k, v, f, W)) / (2 * h)).ravel()
        np.testing.assert_allclose(J, Jfd, rtol=1e-7, atol=1e-9)


def test_backward_state_gradient_is_jacobian_transpose_chain():
    # dH0 = sum_t J_1^T ... J_t^T vec(q_t u_t^T) + J_1^T ... J_T^T vec(dHT), with the dense
    # Jacobians of the pararnn "Jacobian class" remark.
    rng = np.random.default_rng(11)
    B, T, N, K, V = 1, 6, 1, 3, 2
    c = _rand_case(12, B=B, T=T, N=N, K=K, V=V)
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))
    o = oracle.forward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], c["H0"],
                       keep_states=True)
    Js = [oracle.step_jacobian_dense(o["H"][t][0, 0], o["Z"][t][0, 0], c["f"][0, t, 0],
                                     c["W"][0]) for t in range(T)]
    lam = dHT[0, 0].ravel()
    for t in range(T - 1, -1, -1):
        lam = lam + np.outer(c["q"][0, t, 0], dy[0, t, 0]).ravel()
        lam = Js[t].T @ lam
    g = oracle.backward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], dy, c["H0"], dHT)
    np.testing.assert_allclose(g["dH0"][0, 0].ravel(), lam, rtol=1e-12, atol=1e-13)


def _loss(c, dy, dHT, gate_kind, logit, alpha, beta):
    f = oracle.gates(gate_kind, logit, alpha, beta)
    o = oracle.forward(c["k"], c["v"], c["q"], f, c["W"], c["w_r"], c["H0"])
    return float(np.sum(o["y"] * dy) + np.sum(o["HT"] * dHT))


@pytest.mark.parametrize("gate_kind", [GATE_SIGMOID, GATE_EXP_SOFTPLUS])
def test_backward_matches_central_differences(gate_kind):
    # Brute force: every input element, central differences in float64.
    rng = np.random.default_rng(20 + gate_kind)
    B, T, N, K, V = 2, 5, 2, 3, 4
    c = _rand_case(30 + gate_kind, B=B, T=T, N=N, K=K, V=V)
    logit = rng.standard_normal((B, T, N))
    alpha = np.exp(rng.uniform(math.log(0.1), math.log(2.0), N))
    beta = rng.uniform(-2, 2, N)
    if gate_kind == GATE_SIGMOID:
        alpha = beta = None
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))
    f = oracle.gates(gate_kind, logit, alpha, beta)
    g = oracle.backward(c["k"], c["v"], c["q"], f, c["W"], c["w_r"], dy, c["H0"], dHT,
                        gate_kind=gate_kind, logit=logit, alpha=alpha, beta=beta)
    params = {"k": ("dk", c["k"]), "v": ("dv", c["v"]), "q": ("dq", c["q"]),
              "W": ("dW", c["W"]), "w_r": ("dw_r", c["w_r"]), "H0": ("dH0", c["H0"]),
              "logit": ("dlogit", logit)}
    if gate_kind == GATE_EXP_SOFTPLUS:
        params["alpha"] = ("dalpha", alpha)
        params["beta"] = ("dbeta", beta)
    h = 1e-6
    for name, (gname, arr) in params.items():
        fd = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(c, dy, dHT, gate_kind, logit, alpha, beta)
            arr[idx] = old - h
            lm = _loss(c, dy, dHT, gate_kind, logit, alpha, beta)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def _torch_forward(k, v, q, f, W, w_r, H0):
    B, T, N, K = k.shape
    H = H0
    ys = []
    for t in range(T):
        Z = torch.tanh(torch.matmul(H, W[None]) + k[:, t, :, :, None] * v[:, t, :, None, :])
        ft = f[:, t, :, None, None]
        H = ft * H + (1 - ft) * Z
        ys.append(torch.matmul(q[:, t, :, None, :], H)[:, :, 0, :] + w_r[None] * v[:, t])
    return torch.stack(ys, 1), H


@pytest.mark.parametrize("name", ["tiny_fp32", "fp32_k64", "fwd_bwd_k32_v128"])
def test_backward_matches_torch_autograd(name):
    # Autograd of a direct torch transcription of Eq. (10)-(12): an independent
    # differentiation of the same forward, on the recipes of three workloads.
    wl = WORKLOADS[name]
    wl = wl.replace(B=2, T=min(wl.T, 48), N=min(wl.N, 2))
    inp = make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)
    tt = lambda a: torch.from_numpy(np.asarray(a, np.float64).copy()).requires_grad_(True)  # noqa: E731
    k, v, q, W, w_r, H0, logit = map(tt, (inp.k, inp.v, inp.q, inp.W, inp.w_r, inp.H0,
                                         inp.logit))
    if wl.gate == GATE_SIGMOID:
        f = torch.sigmoid(logit)
        alpha = beta = None
    else:
        alpha, beta = tt(inp.alpha), tt(inp.beta)
        f = torch.exp(-alpha * torch.nn.functional.softplus(logit + beta))
    y, HT = _torch_forward(k, v, q, f, W, w_r, H0)
    loss = (y * torch.from_numpy(inp.dy.astype(np.float64))).sum() + \
        (HT * torch.from_numpy(inp.dHT.astype(np.float64))).sum()
    loss.backward()
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    o = oracle.forward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r, inp.H0)
    np.testing.assert_allclose(o["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    g = oracle.backward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r, inp.dy, inp.H0, inp.dHT,
                        gate_kind=wl.gate, logit=inp.logit, alpha=inp.alpha, beta=inp.beta)
    pairs = [("dk", k), ("dv", v), ("dq", q), ("dW", W), ("dw_r", w_r), ("dH0", H0),
             ("dlogit", logit)]
    if alpha is not None:
        pairs += [("dalpha", alpha), ("dbeta", beta)]
    for gname, tens in pairs:
        ref = tens.grad.numpy()
        scale = max(1.0, np.abs(ref).max())
        np.testing.assert_allclose(g[gname], ref, rtol=0, atol=1e-11 * scale, err_msg=gname)


@pytest.mark.parametrize("NQ", [1, 2])
def test_shared_qk_matches_torch_autograd(NQ):
    # q and k shared by groups of N / NQ value heads ([R] section 2.4): torch
    # repeats each shared head over its group and autograd sums the gradient
    # over the group by itself.
    rng = np.random.default_rng(70 + NQ)
    B, T, N, K, V = 2, 9, 4, 3, 5
    c = _rand_case(80 + NQ, B=B, T=T, N=N, K=K, V=V)
    c["k"] = rng.standard_normal((B, T, NQ, K)) * 0.7
    c["q"] = rng.standard_normal((B, T, NQ, K))
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))
    tt = lambda a: torch.from_numpy(np.asarray(a, np.float64).copy()).requires_grad_(True)  # noqa: E731
    k, q, v, f, W, w_r, H0 = map(tt, (c["k"], c["q"], c["v"], c["f"], c["W"], c["w_r"],
                                     c["H0"]))
    y, HT = _torch_forward(torch.repeat_interleave(k, N // NQ, dim=2), v,
                           torch.repeat_interleave(q, N // NQ, dim=2), f, W, w_r, H0)
    loss = (y * torch.from_numpy(dy)).sum() + (HT * torch.from_numpy(dHT)).sum()
    loss.backward()
    o = oracle.forward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], c["H0"])
    np.testing.assert_allclose(o["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o["HT"], HT.detach().numpy(), rtol=1e-12, atol=1e-13)
    g = oracle.backward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], dy, c["H0"], dHT)
    assert g["dk"].shape == (B, T, NQ, K) and g["dq"].shape == (B, T, NQ, K)
    for gname, tens in [("dk", k), ("dq", q), ("dv", v), ("df", f), ("dW", W),
                        ("dw_r", w_r), ("dH0", H0)]:
        ref = tens.grad.numpy()
        np.testing.assert_allclose(g[gname], ref, rtol=0,
                                   atol=1e-11 * max(1.0, np.abs(ref).max()), err_msg=gname)


def test_shared_qk_central_differences():
    # Brute force on the shared operands: every element of a q and k shared by
    # all value heads (NQ = 1), central differences in float64.
    rng = np.random.default_rng(91)
    B, T, N, K, V = 1, 4, 3, 2, 3
    c = _rand_case(92, B=B, T=T, N=N, K=K, V=V)
    c["k"] = rng.standard_normal((B, T, 1, K)) * 0.7
    c["q"] = rng.standard_normal((B, T, 1, K))
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))

    def loss():
        o = oracle.forward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], c["H0"])
        return float(np.sum(o["y"] * dy) + np.sum(o["HT"] * dHT))

    g = oracle.backward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], dy, c["H0"], dHT)
    h = 1e-6
    for name in ("k", "q"):
        arr = c[name]
        fd = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss()
            arr[idx] = old - h
            lm = loss()
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g["d" + name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


# ---------------------------------------------------------------- decode step

def test_decode_step_gate_one_keeps_state_and_reads_it_out():
    # f = 1: H_t = H_{t-1} exactly, and y = H^T q + w_r (.) v by brute-force sums.
    rng = np.random.default_rng(101)
    B, N, K, V = 2, 3, 5, 4
    H = rng.uniform(-0.7, 0.7, (B, N, K, V))
    k, q = rng.standard_normal((B, N, K)), rng.standard_normal((B, N, K))
    v = rng.standard_normal((B, N, V))
    W = rng.standard_normal((N, V, V))
    w_r = rng.standard_normal((N, V))
    Hn, y = oracle.decode_step(H, k, v, q, np.ones((B, N)), W, w_r)
    assert np.array_equal(Hn, H)
    for b in range(B):
        for n in range(N):
            for j in range(V):
                ref = sum(H[b, n, i, j] * q[b, n, i] for i in range(K)) + w_r[n, j] * v[b, n, j]
                assert abs(y[b, n, j] - ref) < 1e-12


def test_decode_step_gate_zero_w_zero_is_tanh_outer():
    rng = np.random.default_rng(102)
    B, N, K, V = 2, 2, 3, 6
    H = rng.uniform(-0.7, 0.7, (B, N, K, V))
    k, q = rng.standard_normal((B, N, K)), rng.standard_normal((B, N, K))
    v = rng.standard_normal((B, N, V))
    Hn, _ = oracle.decode_step(H, k, v, q, np.zeros((B, N)), np.zeros((N, V, V)),
                               np.zeros((N, V)))
    for b in range(B):
        for n in range(N):
            np.testing.assert_allclose(Hn[b, n], np.tanh(np.outer(k[b, n], v[b, n])),
                                       rtol=0, atol=1e-15)


@pytest.mark.parametrize("NQ", [1, 3])
def test_decode_steps_chain_to_the_torch_recurrence(NQ):
    # T decode steps from H_0 reproduce a direct torch transcription of
    # Eq. (10)-(12) over the same T tokens (y at every step and H_T).
    rng = np.random.default_rng(103 + NQ)
    B, T, N, K, V = 2, 6, 3, 4, 5
    c = _rand_case(104, B=B, T=T, N=N, K=K, V=V)
    k = rng.standard_normal((B, T, NQ, K)) * 0.7
    q = rng.standard_normal((B, T, NQ, K))
    H = c["H0"]
    ys = []
    for t in range(T):
        H, y = oracle.decode_step(H, k[:, t], c["v"][:, t], q[:, t], c["f"][:, t], c["W"],
                                  c["w_r"])
        ys.append(y)
    tt = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    G = N // NQ
    yr, HT = _torch_forward(torch.repeat_interleave(tt(k), G, dim=2), tt(c["v"]),
                            torch.repeat_interleave(tt(q), G, dim=2), tt(c["f"]), tt(c["W"]),
                            tt(c["w_r"]), tt(c["H0"]))
    np.testing.assert_allclose(np.stack(ys, 1), yr.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(H, HT.numpy(), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- sensitivity helper

def test_tangent_growth_linear_regime_closed_form():
    # Inputs ~0 keep Z ~ 0, so tanh' ~ 1 and the tangent map is f I + (1-f) c I per step:
    # growth over T steps is (f + (1-f) c)^T when that factor exceeds 1, else 1.
    B, T, N, K, V = 1, 40, 2, 2, 3
    k = np.zeros((B, T, N, K))
    v = np.zeros((B, T, N, V))
    q = np.zeros((B, T, N, K))
    f = np.full((B, T, N), 0.5)
    W = np.stack([1.1 * np.eye(V), 0.7 * np.eye(V)])
    g = oracle.tangent_growth(k, v, q, f, W)
    np.testing.assert_allclose(g[0, 0], (0.5 + 0.5 * 1.1) ** T, rtol=1e-12)
    np.testing.assert_allclose(g[0, 1], 1.0, rtol=0, atol=0)


def _fd_growth(H):
    """max over rows of max_{s <= t} |D_t[i]| / |D_s[i]| (max-abs norm over the
    row) of a state-difference trajectory D [T+1, B, N, K, V], per (b, n)."""
    m = np.abs(H).max(axis=-1)                # [T+1, B, N, K]
    best = np.ones(m.shape[1:])
    run_min = m[0]
    for t in range(1, m.shape[0]):
        best = np.maximum(best, m[t] / run_min)
        run_min = np.minimum(run_min, m[t])
    return best.max(axis=-1)


@pytest.mark.parametrize("seed", [0, 3])
def test_tangent_growth_matches_finite_differences_nonlinear(seed):
    # Nonlinear regime: k, v, H0 of order one keep |A| ~ 1, so 1 - Z^2 is far
    # from 1 and from 0 and varies per element and step.  Two forwards from H0
    # and H0 + eps dH0 (dH0 the tangent's own start: PCG64(seed) normals scaled
    # to max-abs 1 per row) differ by eps J_t...J_1 dH0 + O(eps^2); the
    # per-row growth of that difference must equal tangent_growth's.  A wrong 1 - Z^2
    # factor, a Z taken from the wrong step, or W applied from the wrong side
    # changes the growth by far more than the tolerance.
    rng = np.random.default_rng(11 + seed)
    B, T, N, K, V = 2, 30, 2, 3, 4
    k = rng.standard_normal((B, T, N, K))
    v = rng.standard_normal((B, T, N, V))
    q = rng.standard_normal((B, T, N, K))
    f = rng.uniform(0.2, 0.9, (B, T, N))
    W = np.stack([np.eye(V) + 0.6 * rng.standard_normal((V, V)),
                  1.5 * rng.standard_normal((V, V))])
    H0 = rng.uniform(-0.8, 0.8, (B, N, K, V))
    w_r = np.zeros((N, V))
    g = oracle.tangent_growth(k, v, q, f, W, H0=H0, seed=seed)
    dH = np.random.Generator(np.random.PCG64(seed)).standard_normal((B, N, K, V))
    dH /= np.abs(dH).max(axis=-1)[..., None]
    eps = 1e-6
    Ha = oracle.forward(k, v, q, f, W, w_r, H0=H0 + eps * dH, keep_states=True)["H"]
    Hb = oracle.forward(k, v, q, f, W, w_r, H0=H0 - eps * dH, keep_states=True)["H"]
    g_fd = _fd_growth((Ha - Hb) / (2 * eps))
    assert np.all(g > 1.5), g          # the cases do amplify
    np.testing.assert_allclose(g, g_fd, rtol=1e-6)
