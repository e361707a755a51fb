"""Pins of the float64 parallel-in-time Newton oracle (oracle.newton_forward).

Source: the pararnn-torch "ParaM2RNN" page ("Jacobian class", "Parallel
path": factorized Newton on the matrix residual; "Agreement": compare with the
sequential recurrence) and the "ParaGRU" page ("Parallel path": Newton + scan,
initial guess F(0, x_t), about three iterations).

Each pin ties the Newton oracle to something other than itself: the pinned
sequential forward (oracle.forward), the pinned single step (oracle.decode_step),
central differences of the step map, or a closed property of Newton's method
(exactness on an affine map, causality, a fixed point, quadratic convergence).
"""
import numpy as np
import pytest

import oracle
from m2rnn_inputs import WORKLOADS, make_inputs


def _case(seed, B=2, T=9, N=2, K=3, V=4, W=None, NQ=None):
    rng = np.random.default_rng(seed)
    nq = N if NQ is None else NQ
    c = dict(
        k=rng.standard_normal((B, T, nq, K)) * 0.7,
        v=rng.standard_normal((B, T, N, V)) * 0.7,
        q=rng.standard_normal((B, T, nq, K)),
        f=rng.uniform(0.05, 0.95, (B, T, N)),
        W=(np.eye(V)[None] * 0.8 + rng.standard_normal((N, V, V)) * 0.3) if W is None else W,
        w_r=rng.standard_normal((N, V)) * 0.5,
        H0=rng.uniform(-0.6, 0.6, (B, N, K, V)),
    )
    return c


def _seq(c):
    return oracle.forward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], c["H0"],
                          keep_states=True)


def _newton(c, iters, **kw):
    return oracle.newton_forward(c["k"], c["v"], c["q"], c["f"], c["W"], c["w_r"], c["H0"],
                                 iters=iters, **kw)


@pytest.mark.parametrize("NQ", [None, 1])
def test_newton_is_causal_and_exact_after_T_iterations(NQ):
    # after i iterations the states X_1 .. X_i are the sequential ones (the
    # residual of a causal system is solved one more step per iteration), so
    # T iterations reproduce the forward: states, readouts and H_T
    c = _case(1, NQ=NQ)
    s = _seq(c)
    T = c["v"].shape[1]
    for i in range(T + 1):
        n = _newton(c, i)
        assert np.max(np.abs(n["X"][: i + 1] - s["H"][: i + 1])) < 1e-12, i
    assert np.max(np.abs(n["y"] - s["y"])) < 1e-12
    assert np.max(np.abs(n["X"][T] - s["HT"])) < 1e-12
    assert n["res"][-1] < 1e-12


def test_newton_w_zero_converges_in_one_iteration():
    # with W = 0 the step map is affine in the state, so its linearisation is
    # exact and one Newton step solves the whole sequence
    N, V = 2, 4
    c = _case(2, T=30, W=np.zeros((N, 4, V)))
    n = _newton(c, 1)
    s = _seq(c)
    assert np.max(np.abs(n["X"] - s["H"])) < 1e-12


def test_newton_fixed_point_is_kept():
    # started from the exact states, the residual is zero and so is every update
    c = _case(3, T=25)
    s = _seq(c)
    n = _newton(c, 2, X_init=s["H"])
    assert n["res"][0] < 1e-14
    assert np.max(np.abs(n["X"] - s["H"])) < 1e-14


def test_newton_residual_is_the_step_defect():
    # res[0] is the largest defect X_t - F(X_{t-1}) of the initial guess,
    # F computed by the pinned single step
    c = _case(4, T=12)
    n = _newton(c, 0)
    X = n["X"]
    worst = 0.0
    for t in range(12):
        Ht, _ = oracle.decode_step(X[t], c["k"][:, t], c["v"][:, t], c["q"][:, t], c["f"][:, t],
                                   c["W"], c["w_r"])
        worst = max(worst, float(np.max(np.abs(X[t + 1] - Ht))))
    assert abs(n["res"][0] - worst) < 1e-15
    # the initial guess is F(0, x_t) = (1 - f_t) tanh(k_t v_t^T)
    g = (1 - c["f"][:, 0, :, None, None]) * np.tanh(c["k"][:, 0, :, :, None]
                                                    * c["v"][:, 0, :, None, :])
    assert np.max(np.abs(X[1] - g)) < 1e-15


def test_linearisation_matches_central_differences():
    # J_t h = f h + (1 - f) (h W) (.) s  with s = 1 - Z^2, against
    # (F(X + e h) - F(X - e h)) / 2e of the pinned single step
    rng = np.random.default_rng(5)
    B, N, K, V = 2, 2, 3, 5
    X = rng.uniform(-0.8, 0.8, (B, N, K, V))
    k, v = rng.standard_normal((B, N, K)), rng.standard_normal((B, N, V))
    f = rng.uniform(0.1, 0.9, (B, N))
    W = rng.standard_normal((N, V, V)) * 0.5
    h = rng.standard_normal((B, N, K, V))
    F, s, cc = oracle.newton_linearize(X, k, v, f, W)
    Jh = f[..., None, None] * h + (1 - f[..., None, None]) * np.matmul(h, W[None]) * s
    e = 1e-6
    q0 = np.zeros((B, N, K))
    wr0 = np.zeros((N, V))
    Fp, _ = oracle.decode_step(X + e * h, k, v, q0, f, W, wr0)
    Fm, _ = oracle.decode_step(X - e * h, k, v, q0, f, W, wr0)
    assert np.max(np.abs(Jh - (Fp - Fm) / (2 * e))) < 1e-8
    F0, _ = oracle.decode_step(X, k, v, q0, f, W, wr0)
    assert np.max(np.abs(F - F0)) < 1e-15
    # the affine term: F(X) = J X + c at the linearisation point
    JX = f[..., None, None] * X + (1 - f[..., None, None]) * np.matmul(X, W[None]) * s
    assert np.max(np.abs(JX + cc - F)) < 1e-14


def test_newton_converges_quadratically_on_a_contractive_map():
    # W = 0.9 Q (Q orthogonal): every step Jacobian has norm below 1, and the
    # errors to the sequential states square from one iteration to the next
    wl = WORKLOADS["multi_value_k64_v16"].replace(B=1, T=300, N=2, w_kind="orth",
                                                  w_eps=0.0, w_scale=0.0)
    inp = make_inputs(wl)
    f = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    s = oracle.forward(inp.k, inp.v, inp.q, f, inp.W, inp.w_r, keep_states=True)
    err = []
    for i in range(4):
        n = oracle.newton_forward(inp.k, inp.v, inp.q, f, inp.W, inp.w_r, iters=i)
        err.append(float(np.max(np.abs(n["X"] - s["H"]))))
    assert err[0] > 1e-2
    for i in range(2):
        assert err[i + 1] <= 50 * err[i] ** 2, err
    assert err[3] < 1e-10, err
