"""GPU parity of the single-token step (decoding), m2rnn_step, through the C ABI.

* One step against the float64 oracle's decode step on shapes that span several
  16-row slabs and 16-column tiles with ragged edges, per-head and shared q/k,
  a batch that leaves the last workgroup partial, both state precisions:
  max-abs error 2e-5 (fp32; one step from |H| <= 1 is ~1e-7 off) and 1e-12
  (fp64) on H_t and y.
* T chained steps against the forward kernel over the same T tokens (the two
  sum H W in different orders, so within 2e-5, not bit for bit) and against
  the oracle's forward.
* The scalar-access path: a state tensor that is not 16-byte aligned.
* A batch larger than the device holds workgroups for (several rows per wave,
  a partial last group), and the decode workloads at full size, every unit
  against the oracle.
* Empty calls leave everything untouched.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from m2rnn_inputs import DECODE_WORKLOADS, WORKLOADS, make_inputs, to_device
from matrix_state_nonlinear_amd import m2rnn_fwd, m2rnn_gates, m2rnn_step

pytestmark = pytest.mark.gpu

TOL = {"float32": 2e-5, "float64": 1e-12}


def np_(t):
    return t.detach().cpu().numpy().astype(np.float64)


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def step_case(wl, sd, seed_state=7):
    """Inputs of one decode step: the workload's first token and a random state."""
    inp = make_inputs(wl.replace(T=1))
    rng = np.random.default_rng(seed_state)
    H0 = rng.uniform(-0.9, 0.9, (wl.B, wl.N, wl.K, wl.V))
    d = to_device(inp, sd)
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])[:, 0].contiguous()
    dt = torch.float64 if sd == "float64" else torch.float32
    H = torch.from_numpy(H0).to(dt).to(d["v"].device)
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)[:, 0]
    return inp, d, f, H, H0, fo


def run_step(d, f, H):
    return m2rnn_step(H, d["k"][:, 0].contiguous(), d["v"][:, 0].contiguous(),
                      d["q"][:, 0].contiguous(), f, d["W"], d["w_r"])


SHAPES = [(1, 1), (15, 5), (16, 16), (17, 17), (40, 40), (33, 72), (64, 64), (256, 16),
          (48, 128), (64, 100)]


@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("NQ", [0, 1])
@pytest.mark.parametrize("K,V", SHAPES)
def test_step_matches_oracle(K, V, NQ, sd):
    wl = WORKLOADS["long_t16k_k64"].replace(B=5, N=3, K=K, V=V, NQ=NQ,
                                            kq_scale=1 / math.sqrt(K), v_scale=1 / math.sqrt(V),
                                            w_scale=1 / math.sqrt(V))
    inp, d, f, H, H0, fo = step_case(wl, sd)
    y = run_step(d, f, H)
    torch.cuda.synchronize()
    Hn, yo = oracle.decode_step(H0, inp.k[:, 0], inp.v[:, 0], inp.q[:, 0], fo, inp.W, inp.w_r)
    eh, ey = maxerr(np_(H), Hn), maxerr(np_(y), yo)
    print(f"K={K} V={V} NQ={wl.qk_heads} {sd}: H {eh:.1e} y {ey:.1e}")
    assert eh <= TOL[sd] and ey <= TOL[sd]


@pytest.mark.parametrize("sd", ["float32", "float64"])
@pytest.mark.parametrize("name", ["long_t16k_k64", "multi_value_k64_v16", "fwd_bwd_k32_v128"])
def test_chained_steps_equal_the_forward(name, sd):
    wl = WORKLOADS[name].replace(B=3, T=100, N=min(WORKLOADS[name].N, 4))
    inp = make_inputs(wl, with_h0=True)
    d = to_device(inp, sd)
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
    y_fwd, HT_fwd, _ = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"])
    H = d["H0"].clone()
    ys = []
    for t in range(wl.T):
        ys.append(m2rnn_step(H, d["k"][:, t].contiguous(), d["v"][:, t].contiguous(),
                             d["q"][:, t].contiguous(), f[:, t].contiguous(), d["W"], d["w_r"]))
    torch.cuda.synchronize()
    y_steps = torch.stack(ys, 1)
    fo = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
    o = oracle.forward(inp.k, inp.v, inp.q, fo, inp.W, inp.w_r, inp.H0)
    e_fwd = max(maxerr(np_(y_steps), np_(y_fwd)), maxerr(np_(H), np_(HT_fwd)))
    e_or = max(maxerr(np_(y_steps), o["y"]), maxerr(np_(H), o["HT"]))
    print(f"{name} {sd}: steps vs forward {e_fwd:.1e}, vs oracle {e_or:.1e}")
    assert e_fwd <= TOL[sd] and e_or <= TOL[sd]


def test_step_unaligned_state_takes_the_scalar_path():
    wl = WORKLOADS["long_t16k_k64"].replace(B=5, N=2)
    inp, d, f, H, H0, fo = step_case(wl, "float32")
    buf = torch.empty(H.numel() + 1, dtype=H.dtype, device=H.device)
    Hu = buf[1:].view(H.shape)
    assert Hu.data_ptr() % 16 != 0
    Hu.copy_(H)
    y = run_step(d, f, Hu)
    y_al = run_step(d, f, H)
    torch.cuda.synchronize()
    assert torch.equal(Hu, H) and torch.equal(y, y_al)
    Hn, yo = oracle.decode_step(H0, inp.k[:, 0], inp.v[:, 0], inp.q[:, 0], fo, inp.W, inp.w_r)
    assert maxerr(np_(Hu), Hn) <= TOL["float32"] and maxerr(np_(y), yo) <= TOL["float32"]


@pytest.mark.parametrize("K,V,NQ,B", [(64, 64, 0, 37), (16, 64, 0, 5), (48, 64, 1, 37),
                                      (256, 64, 0, 9), (64, 64, 1, 4099)])
@pytest.mark.parametrize("in_bf16", [True, False])
def test_step_full_tile_kernel_equals_the_general_one(K, V, NQ, B, in_bf16):
    """K a multiple of 16, V = 64 and aligned buffers take the full-tile kernel
    (its LDS ring of state slabs); a y buffer one float off alignment sends the
    same call to the general kernel, whose arithmetic (and order) it shares:
    equal bit for bit.  Batch sizes with one slab per wave (K = 16, B = 5),
    several batch rows per wave and a partial last group (B = 4099)."""
    N = 4 if NQ else 3
    wl = WORKLOADS["long_t16k_k64"].replace(B=B, N=N, NQ=NQ, K=K, V=V, bf16=in_bf16,
                                            kq_scale=1 / math.sqrt(K), v_scale=1 / math.sqrt(V),
                                            w_scale=1 / math.sqrt(V))
    inp, d, f, H, H0, fo = step_case(wl, "float32")
    H2 = H.clone()
    args = (d["k"][:, 0].contiguous(), d["v"][:, 0].contiguous(), d["q"][:, 0].contiguous(), f,
            d["W"], d["w_r"])
    y = m2rnn_step(H, *args)
    buf = torch.empty(y.numel() + 1, dtype=y.dtype, device=y.device)
    y2 = buf[1:].view(y.shape)
    assert y.data_ptr() % 16 == 0 and y2.data_ptr() % 16 != 0
    m2rnn_step(H2, *args, out=y2)
    torch.cuda.synchronize()
    assert torch.equal(H, H2) and torch.equal(y, y2)
    Hn, yo = oracle.decode_step(H0, inp.k[:, 0], inp.v[:, 0], inp.q[:, 0], fo, inp.W, inp.w_r)
    assert maxerr(np_(H), Hn) <= TOL["float32"] and maxerr(np_(y), yo) <= TOL["float32"]


@pytest.mark.parametrize("K,V", [(20, 24), (64, 64)])
def test_step_large_ragged_batch(K, V):
    # more batch rows than the device holds workgroups for: every wave takes
    # several rows in turn, and the last group of four is partial (B % 4 = 3)
    wl = WORKLOADS["long_t16k_k64"].replace(B=4099, N=8, K=K, V=V, kq_scale=1 / math.sqrt(K),
                                            v_scale=1 / math.sqrt(V), w_scale=1 / math.sqrt(V))
    inp, d, f, H, H0, fo = step_case(wl, "float32")
    y = run_step(d, f, H)
    torch.cuda.synchronize()
    Hn, yo = oracle.decode_step(H0, inp.k[:, 0], inp.v[:, 0], inp.q[:, 0], fo, inp.W, inp.w_r)
    eh, ey = maxerr(np_(H), Hn), maxerr(np_(y), yo)
    print(f"B=4099 K={K} V={V}: H {eh:.1e} y {ey:.1e}")
    assert eh <= TOL["float32"] and ey <= TOL["float32"]


@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_workload_full_size(name):
    wl = DECODE_WORKLOADS[name]
    inp, d, f, H, H0, fo = step_case(wl, "float32")
    y = run_step(d, f, H)
    torch.cuda.synchronize()
    Hn, yo = oracle.decode_step(H0, inp.k[:, 0], inp.v[:, 0], inp.q[:, 0], fo, inp.W, inp.w_r)
    eh, ey = maxerr(np_(H), Hn), maxerr(np_(y), yo)
    print(f"{name}: H {eh:.1e} y {ey:.1e}")
    # bf16 inputs are exact on both sides: one fp32 step, far inside the stated 2e-2
    assert eh <= TOL["float32"] and ey <= TOL["float32"]


@pytest.mark.parametrize("B,N", [(0, 3), (4, 0)])
def test_step_empty(B, N):
    wl = WORKLOADS["long_t16k_k64"].replace(B=B, N=N, K=20, V=24)
    inp, d, f, H, H0, fo = step_case(wl, "float32")
    y = run_step(d, f, H)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (B, N, 24) and tuple(H.shape) == (B, N, 20, 24)
