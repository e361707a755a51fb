"""m2rnn_bwd_noalloc (the backward in the library's static per-device scratch)
against m2rnn_bwd (caller's workspace), through the C ABI.

Two calls in a row, the second with a smaller problem than the first, so the
second finds the first's partial sums in the scratch: both must equal
m2rnn_bwd's results bit for bit (same kernels, same order of every sum), in
both backward modes (states recomputed, and read from the stored rc) and with
q/k shared across heads.  A call whose workspace exceeds the scratch is
refused with M2RNN_ERR_SCRATCH before anything runs.
"""
import math

import pytest
import torch

from m2rnn_inputs import WORKLOADS, make_inputs, to_device
from matrix_state_nonlinear_amd import (M2RNNError, m2rnn_fwd, m2rnn_gates,
                                        m2rnn_workspace_bytes)
from matrix_state_nonlinear_amd import _lib
from matrix_state_nonlinear_amd import m2rnn_bwd, m2rnn_bwd_noalloc

pytestmark = pytest.mark.gpu


def _case(B, T, N, K, V, NQ, C, seed):
    wl = WORKLOADS["fwd_bwd_k32_v128"].replace(B=B, T=T, N=N, K=K, V=V, NQ=NQ, seed=seed,
                                               kq_scale=1 / math.sqrt(K),
                                               v_scale=1 / math.sqrt(V), w_scale=1 / math.sqrt(V))
    inp = make_inputs(wl, with_dy=True, with_h0=True, with_dht=True)
    d = to_device(inp, "float32")
    f = m2rnn_gates(d["logit"], wl.gate, d["alpha"], d["beta"])
    rc = torch.empty((B, N, T, K, V), dtype=torch.float32, device=f.device)
    _, _, ck = m2rnn_fwd(d["k"], d["v"], d["q"], f, d["W"], d["w_r"], d["H0"], C, rc_out=rc)
    args = (d["k"], d["v"], d["q"], wl.gate, d["logit"], d["alpha"], d["beta"], f, d["W"],
            d["w_r"], d["H0"], ck, C, d["dy"], d["dHT"])
    return wl, args, rc


# (B, T, N, K, V, NQ, C): the first larger than the second; C = 7 and 5 do not
# divide the backward's chunk length (chunk starts go through the scratch)
FIRST = (2, 70, 4, 40, 72, 2, 7)
SECOND = (1, 33, 2, 17, 40, 1, 5)


@pytest.mark.parametrize("use_rc", [False, True])
def test_noalloc_backward_equals_workspace_backward_twice(use_rc):
    for label, shape in (("first", FIRST), ("second, smaller", SECOND)):
        wl, args, rc = _case(*shape, seed=21 + len(label))
        B, T, N, K, V, NQ, C = shape
        need = m2rnn_workspace_bytes(True, B, T, N, NQ, K, V, C, torch.float32)
        assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES
        ref = m2rnn_bwd(*args, rc=rc if use_rc else None)
        got = m2rnn_bwd_noalloc(*args, rc=rc if use_rc else None)
        torch.cuda.synchronize()
        for name, r in ref.items():
            if r is None:
                assert got[name] is None, name
                continue
            assert torch.equal(r, got[name]), (label, name)
        print(f"{label} call {shape}, rc={use_rc}: bitwise equal to m2rnn_bwd "
              f"(workspace {need} bytes)")


def test_noalloc_refuses_calls_beyond_the_scratch():
    # B * T * N * V * nslab * 4 bytes of dv partials alone exceed 64 MiB
    shape = (1, 4096, 16, 48, 128, 16, 64)
    B, T, N, K, V, NQ, C = shape
    need = m2rnn_workspace_bytes(True, B, T, N, NQ, K, V, C, torch.float32)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    wl, args, _ = _case(*shape, seed=31)
    sentinel = torch.full((B, T, N, V), 7.0, dtype=torch.float32, device="cuda:0")
    with pytest.raises(M2RNNError) as e:
        m2rnn_bwd_noalloc(*args, out={"dv": sentinel})
    assert e.value.status == _lib.M2RNN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all())   # nothing was launched
    print(f"refused: workspace {need} bytes > {_lib.NOALLOC_SCRATCH_BYTES}")
