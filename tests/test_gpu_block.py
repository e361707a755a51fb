"""GPU parity of the block prologue (causal conv + SiLU) and epilogue
(gate + RMSNorm) against the float64 oracle, through the C ABI (review of
"M²RNN: Non-Linear RNNs with Matrix-Valued States for Scalable Language
Modeling", section 2.3).

Tolerances.  Outputs stored as bf16 are rounded once to nearest even from an
fp32 value within ~1e-6 relative of the exact one, so they are within one bf16
unit in the last place of the exact value: |out - ref| <= 2^-8 |ref| + 1e-6.
fp32 outputs and gradients: 1e-5 relative to max(1, max |ref|) per tensor
(parameter gradients sum B T products: 1e-4); fp64: 1e-12.  Shapes cover time
runs of 64 steps with ragged ends, sequences shorter than the kernel, channel
blocks of 256 with ragged ends, and the sizes of the long-context workload
(B = 4, T = 16384, 16 heads x 64 channels) on sampled channels and rows.
"""
import numpy as np
import pytest
import torch

import oracle
from m2rnn_inputs import make_conv_inputs, make_norm_inputs
from matrix_state_nonlinear_amd import (m2rnn_conv_silu, m2rnn_conv_silu_bwd,
                                        m2rnn_gate_rmsnorm, m2rnn_gate_rmsnorm_bwd)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def np_(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 \
        else t.detach().cpu().numpy().astype(np.float64)


def dev_io(values, bits, io):
    """An input in the io dtype: bf16 from its exact bit patterns, else float."""
    if io == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    dt = torch.float64 if io == "f64" else torch.float32
    return torch.from_numpy(np.asarray(values, np.float64)).to(dt).to(DEV)


def param_dtype(io, sd):
    return torch.float64 if sd == "f64" else torch.float32


def dev_p(a, pdt):
    return None if a is None else torch.from_numpy(np.asarray(a, np.float64)).to(pdt).to(DEV)


def check_io_out(out, ref, io):
    got = np_(out)
    if io == "bf16":
        bound = 2.0 ** -8 * np.abs(ref) + 1e-6
        assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) - bound))
    else:
        tol = 1e-12 if io == "f64" else 1e-5
        assert float(np.max(np.abs(got - ref))) <= tol * max(1.0, float(np.max(np.abs(ref))))


def check_grad(g, ref, sd, tau32, name):
    tol = 1e-12 if sd == "f64" else tau32
    err = float(np.max(np.abs(np_(g) - ref))) / max(1.0, float(np.max(np.abs(ref))))
    assert err <= tol, (name, err)
    return err


COMBOS = [("f32", "f32"), ("bf16", "f32"), ("f64", "f64"), ("bf16", "f64")]


@pytest.mark.parametrize("io,sd", COMBOS)
@pytest.mark.parametrize("B,T,C", [(2, 1, 5), (2, 3, 7), (3, 70, 300), (1, 129, 64),
                                   (2, 200, 1030)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_conv_silu_forward_and_backward(B, T, C, io, sd, with_bias):
    inp = make_conv_inputs(B, T, C, seed=B * 1000 + T + C, bf16=(io == "bf16"))
    pdt = param_dtype(io, sd)
    x = dev_io(inp.x, inp.x_bits, io)
    w, bias = dev_p(inp.w, pdt), dev_p(inp.bias if with_bias else None, pdt)
    out = m2rnn_conv_silu(x, w, bias)
    dx, dw, db = m2rnn_conv_silu_bwd(x, w, bias, dev_p(inp.dout, pdt))
    torch.cuda.synchronize()
    b_np = inp.bias if with_bias else None
    check_io_out(out, oracle.conv_silu(inp.x, inp.w, b_np), io)
    rdx, rdw, rdb = oracle.conv_silu_backward(inp.x, inp.w, b_np, inp.dout)
    e = [check_grad(dx, rdx, sd, 1e-5, "dx"), check_grad(dw, rdw, sd, 1e-4, "dw")]
    if with_bias:
        e.append(check_grad(db, rdb, sd, 1e-4, "dbias"))
    else:
        assert db is None
    print(f"B={B} T={T} C={C} {io}/{sd} bias={with_bias}: grads {[f'{v:.1e}' for v in e]}")


@pytest.mark.parametrize("io,sd", COMBOS)
@pytest.mark.parametrize("rows,D", [(1, 1), (7, 24), (300, 1024), (65, 100), (5, 3000)])
def test_gate_rmsnorm_forward_and_backward(rows, D, io, sd):
    inp = make_norm_inputs(rows, D, seed=rows * 7 + D, bf16=(io == "bf16"))
    pdt = param_dtype(io, sd)
    eps = 1e-6
    y, gamma = dev_p(inp.y, pdt), dev_p(inp.gamma, pdt)
    g = dev_io(inp.g_pre, inp.g_bits, io)
    out = m2rnn_gate_rmsnorm(y, g, gamma, eps)
    dy, dg, dgamma = m2rnn_gate_rmsnorm_bwd(y, g, gamma, dev_p(inp.dout, pdt), eps)
    torch.cuda.synchronize()
    check_io_out(out, oracle.gate_rmsnorm(inp.y, inp.g_pre, inp.gamma, eps), io)
    rdy, rdg, rdgamma = oracle.gate_rmsnorm_backward(inp.y, inp.g_pre, inp.gamma, eps, inp.dout)
    e = [check_grad(dy, rdy, sd, 1e-5, "dy"), check_grad(dg, rdg, sd, 1e-5, "dg_pre"),
         check_grad(dgamma, rdgamma, sd, 1e-4, "dgamma")]
    print(f"rows={rows} D={D} {io}/{sd}: grads {[f'{v:.1e}' for v in e]}")


def test_block_deterministic():
    inp = make_conv_inputs(2, 300, 520, seed=5)
    x = dev_io(inp.x, inp.x_bits, "bf16")
    w, bias, dout = (dev_p(a, torch.float32) for a in (inp.w, inp.bias, inp.dout))
    a = m2rnn_conv_silu_bwd(x, w, bias, dout)
    b = m2rnn_conv_silu_bwd(x, w, bias, dout)
    assert all(torch.equal(p, q) for p, q in zip(a, b))


def test_block_full_size_long_context():
    """The v prologue and the epilogue at the long-context workload's sizes
    (B = 4, T = 16384, C = D = 16 x 64 = 1024): conv outputs and dx on two
    channel slices (each channel is independent), dw and dbias of those
    channels (full sums), the epilogue and its row gradients on 512 rows, and
    dgamma against the oracle over all rows."""
    B, T, C = 4, 16384, 1024
    inp = make_conv_inputs(B, T, C, seed=21)
    x = dev_io(inp.x, inp.x_bits, "bf16")
    w, bias, dout = (dev_p(a, torch.float32) for a in (inp.w, inp.bias, inp.dout))
    out = m2rnn_conv_silu(x, w, bias)
    dx, dw, db = m2rnn_conv_silu_bwd(x, w, bias, dout)
    torch.cuda.synchronize()
    for sl in (slice(0, 48), slice(1000, 1024)):
        ref = oracle.conv_silu(inp.x[:, :, sl], inp.w[sl], inp.bias[sl])
        check_io_out(out[:, :, sl], ref, "bf16")
        rdx, rdw, rdb = oracle.conv_silu_backward(inp.x[:, :, sl], inp.w[sl], inp.bias[sl],
                                                  inp.dout[:, :, sl])
        check_grad(dx[:, :, sl], rdx, "f32", 1e-5, "dx")
        check_grad(dw[sl], rdw, "f32", 1e-4, "dw")
        check_grad(db[sl], rdb, "f32", 1e-4, "dbias")
    del x, out, dx
    rows, D = B * T, C
    ninp = make_norm_inputs(rows, D, seed=22)
    y, gamma, nd = (dev_p(a, torch.float32) for a in (ninp.y, ninp.gamma, ninp.dout))
    g = dev_io(ninp.g_pre, ninp.g_bits, "bf16")
    o = m2rnn_gate_rmsnorm(y, g, gamma, 1e-6)
    dy, dg, dgamma = m2rnn_gate_rmsnorm_bwd(y, g, gamma, nd, 1e-6)
    torch.cuda.synchronize()
    rs = np.random.default_rng(23).choice(rows, 512, replace=False)
    check_io_out(o[rs], oracle.gate_rmsnorm(ninp.y[rs], ninp.g_pre[rs], ninp.gamma, 1e-6), "bf16")
    rdy, rdg, _ = oracle.gate_rmsnorm_backward(ninp.y[rs], ninp.g_pre[rs], ninp.gamma, 1e-6,
                                               ninp.dout[rs])
    check_grad(dy[rs], rdy, "f32", 1e-5, "dy")
    check_grad(dg[rs], rdg, "f32", 1e-5, "dg_pre")
    _, _, rdgamma = oracle.gate_rmsnorm_backward(ninp.y, ninp.g_pre, ninp.gamma, 1e-6,
                                                 ninp.dout)
    check_grad(dgamma, rdgamma, "f32", 1e-4, "dgamma")
