"""Pins of the oracle's block prologue / epilogue (review of "M²RNN: Non-Linear
RNNs with Matrix-Valued States for Scalable Language Modeling", section 2.3):
the causal convolution against torch's depthwise conv1d, SiLU against torch,
RMSNorm against torch's rms_norm, both backwards against torch autograd, and
closed-form special cases.  None compares the oracle with itself."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _t(a, grad=False):
    return torch.from_numpy(np.asarray(a, np.float64).copy()).requires_grad_(grad)


def _torch_conv_silu(x, w, bias):
    # depthwise causal conv: left padding 3, groups = channels, the first T outputs
    B, T, C = x.shape
    u = F.conv1d(x.transpose(1, 2), w[:, None, :], bias, padding=w.shape[1] - 1, groups=C)
    return F.silu(u[:, :, :T].transpose(1, 2))


@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 11])
def test_conv_silu_matches_torch_conv1d(T, with_bias):
    rng = np.random.default_rng(200 + T)
    B, C = 3, 7
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, 4)) * 0.6
    bias = rng.standard_normal(C) * 0.3 if with_bias else None
    ref = _torch_conv_silu(_t(x), _t(w), None if bias is None else _t(bias)).numpy()
    np.testing.assert_allclose(oracle.conv_silu(x, w, bias), ref, rtol=0, atol=1e-14)


def test_conv_last_tap_only_is_identity_and_silu_matches_torch():
    rng = np.random.default_rng(210)
    x = rng.standard_normal((2, 9, 5)) * 30  # large |x|: both sigmoid branches
    w = np.zeros((5, 4))
    w[:, 3] = 1.0
    assert np.array_equal(oracle.causal_conv(x, w), x)
    np.testing.assert_allclose(oracle.conv_silu(x, w), F.silu(_t(x)).numpy(), rtol=1e-15,
                               atol=1e-300)


def test_silu_grad_matches_autograd():
    x = _t(np.linspace(-40, 40, 801), grad=True)
    F.silu(x).sum().backward()
    np.testing.assert_allclose(oracle.silu_grad(x.detach().numpy()), x.grad.numpy(),
                               rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("with_bias", [True, False])
def test_conv_silu_backward_matches_autograd(with_bias):
    rng = np.random.default_rng(220)
    B, T, C = 2, 13, 6
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal((C, 4)) * 0.6
    bias = rng.standard_normal(C) * 0.3 if with_bias else None
    dout = rng.standard_normal((B, T, C))
    xt, wt = _t(x, True), _t(w, True)
    bt = None if bias is None else _t(bias, True)
    (_torch_conv_silu(xt, wt, bt) * _t(dout)).sum().backward()
    dx, dw, db = oracle.conv_silu_backward(x, w, bias, dout)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=0, atol=1e-12)
    if with_bias:
        np.testing.assert_allclose(db, bt.grad.numpy(), rtol=0, atol=1e-12)
    else:
        assert db is None


def test_gate_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(230)
    B, T, D = 2, 5, 24
    y = rng.standard_normal((B, T, D))
    g_pre = rng.standard_normal((B, T, D)) * 2
    gamma = rng.uniform(0.5, 1.5, D)
    eps = 1e-6
    z = _t(y) * F.silu(_t(g_pre))
    ref = F.rms_norm(z, (D,), weight=_t(gamma), eps=eps).numpy()
    np.testing.assert_allclose(oracle.gate_rmsnorm(y, g_pre, gamma, eps), ref, rtol=1e-13,
                               atol=1e-14)


def test_rmsnorm_of_a_constant_row_is_its_sign():
    # z = c (all channels equal): z / rms(z) = sign(c) exactly when eps = 0
    D = 10
    y = np.array([[[0.3] * D, [-2.0] * D]])
    g_pre = np.full((1, 2, D), 50.0)  # SiLU(50) = 50 (1 - 2e-22): sigmoid rounds to 1
    out = oracle.gate_rmsnorm(y, g_pre, np.ones(D), 0.0)
    np.testing.assert_allclose(out[0, 0], 1.0, rtol=1e-15)
    np.testing.assert_allclose(out[0, 1], -1.0, rtol=1e-15)


def test_gate_rmsnorm_backward_matches_autograd():
    rng = np.random.default_rng(240)
    B, T, D = 3, 4, 20
    y = rng.standard_normal((B, T, D))
    g_pre = rng.standard_normal((B, T, D)) * 2
    gamma = rng.uniform(0.5, 1.5, D)
    dout = rng.standard_normal((B, T, D))
    eps = 1e-5
    yt, gt, wt = _t(y, True), _t(g_pre, True), _t(gamma, True)
    (F.rms_norm(yt * F.silu(gt), (D,), weight=wt, eps=eps) * _t(dout)).sum().backward()
    dy, dg, dgamma = oracle.gate_rmsnorm_backward(y, g_pre, gamma, eps, dout)
    np.testing.assert_allclose(dy, yt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dgamma, wt.grad.numpy(), rtol=0, atol=1e-12)
