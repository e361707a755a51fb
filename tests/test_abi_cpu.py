"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library loads, exports every function include/m2rnn.h declares, sizes its
workspace as documented, and rejects bad arguments with the documented status
before any launch (every case below fails a host-side check).
"""
import os
import re

import pytest

from matrix_state_nonlinear_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: every call below is rejected on the host


def header_functions():
    src = open(os.path.join(ROOT, "include", "m2rnn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(m2rnn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from matrix_state_nonlinear_amd import build
        build.build()
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert names == sorted(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(6):
        assert _lib.status_string(s).startswith("M2RNN")
    assert "unknown" in _lib.status_string(99)


def test_workspace_sizes(L):
    ws = L.m2rnn_workspace_bytes
    # one slab per head: no forward workspace
    assert ws(0, 2, 64, 1, 1, 8, 8, 1, _lib.M2RNN_F32) == 0
    # K = 64 -> 4 slabs of partial readouts
    b = ws(0, 4, 100, 3, 3, 64, 40, 1, _lib.M2RNN_F32)
    assert b == ((4 * 4 * 100 * 3 * 40 * 4 + 255) // 256) * 256
    assert ws(0, 4, 100, 3, 3, 64, 40, 1, _lib.M2RNN_F64) == ((4 * 4 * 100 * 3 * 40 * 8 + 255) // 256) * 256
    # unsupported sizes report 0
    assert ws(0, 1, 10, 1, 1, 300, 16, 1, _lib.M2RNN_F32) == 0
    assert ws(1, 1, 10, 1, 1, 16, 16, 0, _lib.M2RNN_F32) == 0
    # backward: for V = 64 in fp32 the reverse sweep walks 4-step chunks; a
    # checkpoint interval dividing 4 provides every chunk start; any other adds
    # a [B, N, ceil(T / 4), K, V] region of recomputed chunk starts
    base = ws(1, 2, 64, 2, 2, 32, 64, 4, _lib.M2RNN_F32)
    assert base > 0
    for C in (1, 2):
        assert ws(1, 2, 64, 2, 2, 32, 64, C, _lib.M2RNN_F32) == base
    for C in (3, 6, 8, 64, 1024, 2048):
        assert ws(1, 2, 64, 2, 2, 32, 64, C, _lib.M2RNN_F32) == base + 2 * 2 * 16 * 32 * 64 * 4
    # at V = 128 (2-step chunks) a larger multiple of 2, up to 1024, is swept by
    # the main kernel, which keeps two intervals of states and of rc per 16-row
    # slab ([units, 2, C, 16, 128] each); odd intervals and longer ones take the
    # chunk-start region [B, N, ceil(T / 2), K, V]
    base = ws(1, 2, 64, 2, 2, 32, 128, 2, _lib.M2RNN_F32)
    assert base > 0
    assert ws(1, 2, 64, 2, 2, 32, 128, 1, _lib.M2RNN_F32) == base
    for C in (3, 2048):
        assert ws(1, 2, 64, 2, 2, 32, 128, C, _lib.M2RNN_F32) == base + 2 * 2 * 32 * 32 * 128 * 4
    units = 2 * 2 * 2
    for C in (4, 64, 1024):
        assert ws(1, 2, 64, 2, 2, 32, 128, C, _lib.M2RNN_F32) == \
            base + 2 * units * 2 * C * 16 * 128 * 4


def fwd(L, **kw):
    a = dict(B=2, T=8, N=1, NQ=None, K=16, V=16, ind=_lib.M2RNN_F32, sd=_lib.M2RNN_F32, k=FAKE,
             v=FAKE, q=FAKE, f=FAKE, W=FAKE, w_r=FAKE, H0=None, y=FAKE, HT=None, ckpt=None, C=0,
             rc=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    if a["NQ"] is None:
        a["NQ"] = a["N"]
    return L.m2rnn_fwd(a["B"], a["T"], a["N"], a["NQ"], a["K"], a["V"], a["ind"], a["sd"], a["k"], a["v"],
                       a["q"], a["f"], a["W"], a["w_r"], a["H0"], a["y"], a["HT"], a["ckpt"],
                       a["C"], a["rc"], a["ws"], a["wsb"], a["stream"])


def test_qk_heads_must_divide_n_heads(L):
    """q and k have qk_heads heads shared by groups of n_heads / qk_heads value
    heads: qk_heads divides n_heads; both are 0 only when there are no heads."""
    E = _lib
    for N, NQ in ((4, 0), (4, 3), (4, 5), (4, -1), (0, 1), (6, 4)):
        assert fwd(L, N=N, NQ=NQ) == E.M2RNN_ERR_INVALID_ARG, (N, NQ)
        assert bwd(L, N=N, NQ=NQ) == E.M2RNN_ERR_INVALID_ARG, (N, NQ)
        assert L.m2rnn_workspace_bytes(1, 2, 8, N, NQ, 16, 16, 4, E.M2RNN_F32) == 0, (N, NQ)
    assert fwd(L, N=0, NQ=0, k=None, v=None, q=None, f=None, W=None, w_r=None,
               y=None) == E.M2RNN_OK
    # shared heads: the backward keeps per-value-head dk and dq partials
    # ([B, T, n_heads, K] each) that are summed over the groups
    for NQ in (1, 2):
        extra = L.m2rnn_workspace_bytes(1, 2, 64, 4, NQ, 32, 64, 4, E.M2RNN_F32) - \
            L.m2rnn_workspace_bytes(1, 2, 64, 4, 4, 32, 64, 4, E.M2RNN_F32)
        assert extra == 2 * 2 * 64 * 4 * 32 * 4
    assert L.m2rnn_workspace_bytes(0, 2, 64, 4, 1, 32, 64, 4, E.M2RNN_F32) == \
        L.m2rnn_workspace_bytes(0, 2, 64, 4, 4, 32, 64, 4, E.M2RNN_F32)


def test_fwd_rejects_bad_arguments(L):
    E = _lib
    assert fwd(L, B=-1) == E.M2RNN_ERR_INVALID_ARG
    assert fwd(L, T=-1) == E.M2RNN_ERR_INVALID_ARG
    assert fwd(L, K=0) == E.M2RNN_ERR_INVALID_ARG
    assert fwd(L, V=0) == E.M2RNN_ERR_INVALID_ARG
    assert fwd(L, k=None) == E.M2RNN_ERR_INVALID_ARG
    assert fwd(L, y=None) == E.M2RNN_ERR_INVALID_ARG
    assert fwd(L, ckpt=FAKE, C=0) == E.M2RNN_ERR_INVALID_ARG
    assert fwd(L, ind=7) == E.M2RNN_ERR_INVALID_ARG
    assert fwd(L, K=257) == E.M2RNN_ERR_UNSUPPORTED
    assert fwd(L, V=129) == E.M2RNN_ERR_UNSUPPORTED
    assert fwd(L, ind=E.M2RNN_F64) == E.M2RNN_ERR_UNSUPPORTED          # f64 inputs, f32 state
    assert fwd(L, sd=E.M2RNN_F64, ind=E.M2RNN_F32) == E.M2RNN_ERR_UNSUPPORTED
    assert fwd(L, K=64) == E.M2RNN_ERR_WORKSPACE                       # needs partials
    assert fwd(L, K=64, ws=FAKE, wsb=16) == E.M2RNN_ERR_WORKSPACE


def test_empty_calls_need_no_pointers_or_workspace(L):
    """An empty batch or sequence is a defined call: the per-token arrays may be
    NULL and no workspace is needed; with no state or per-head output to
    write (HT, dH0 NULL, no heads) nothing is launched and the call succeeds
    here, without a GPU."""
    E = _lib
    assert L.m2rnn_workspace_bytes(1, 0, 8, 2, 2, 16, 16, 4, E.M2RNN_F32) == 0
    assert L.m2rnn_workspace_bytes(0, 2, 0, 2, 2, 64, 16, 4, E.M2RNN_F32) == 0
    assert fwd(L, B=0, k=None, v=None, q=None, f=None, W=None, w_r=None, y=None,
               HT=None, ckpt=None) == E.M2RNN_OK
    assert fwd(L, T=0, K=64, HT=None, ckpt=FAKE, C=4) == E.M2RNN_OK
    g = L.m2rnn_gates
    assert g(2, 0, 2, E.M2RNN_GATE_SIGMOID, E.M2RNN_F32, None, None, None, None, None) == E.M2RNN_OK
    assert g(2, 0, 2, E.M2RNN_GATE_EXP_SOFTPLUS, E.M2RNN_F32, None, None, None, None, None) == E.M2RNN_OK
    assert bwd(L, N=0, k=None, v=None, q=None, logit=None, f=None, W=None, w_r=None, ckpt=None,
               dy=None, dk=None, dv=None, dq=None, dlogit=None, dW=None, dw_r=None) == E.M2RNN_OK
    # with heads, dW and dw_r are required (they are written even for no tokens)
    assert bwd(L, T=0, dW=None) == E.M2RNN_ERR_INVALID_ARG
    assert bwd(L, B=-1) == E.M2RNN_ERR_INVALID_ARG


def test_gates_rejects_bad_arguments(L):
    E = _lib
    g = L.m2rnn_gates
    assert g(-1, 4, 2, E.M2RNN_GATE_SIGMOID, E.M2RNN_F32, FAKE, None, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert g(1, 4, 2, E.M2RNN_GATE_SIGMOID, E.M2RNN_F32, FAKE, FAKE, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert g(1, 4, 2, E.M2RNN_GATE_EXP_SOFTPLUS, E.M2RNN_F32, FAKE, None, FAKE, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert g(1, 4, 2, 5, E.M2RNN_F32, FAKE, None, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert g(1, 4, 2, E.M2RNN_GATE_SIGMOID, E.M2RNN_BF16, FAKE, None, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert g(1, 4, 2, E.M2RNN_GATE_SIGMOID, E.M2RNN_F32, None, None, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG


def bwd(L, **kw):
    a = dict(B=2, T=8, N=1, NQ=None, K=16, V=16, ind=_lib.M2RNN_F32, sd=_lib.M2RNN_F32, k=FAKE, v=FAKE,
             q=FAKE, gate=_lib.M2RNN_GATE_SIGMOID, logit=FAKE, alpha=None, beta=None, f=FAKE,
             W=FAKE, w_r=FAKE, H0=None, ckpt=FAKE, C=4, rc=None, dy=FAKE, dHT=None, dk=FAKE,
             dv=FAKE,
             dq=FAKE, dlogit=FAKE, dW=FAKE, dw_r=FAKE, dalpha=None, dbeta=None, dH0=None,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    if a["NQ"] is None:
        a["NQ"] = a["N"]
    keys = ["B", "T", "N", "NQ", "K", "V", "ind", "sd", "k", "v", "q", "gate", "logit", "alpha", "beta",
            "f", "W", "w_r", "H0", "ckpt", "C", "rc", "dy", "dHT", "dk", "dv", "dq", "dlogit", "dW",
            "dw_r", "dalpha", "dbeta", "dH0", "ws", "wsb", "stream"]
    return L.m2rnn_bwd(*[a[k] for k in keys])


def test_bwd_rejects_bad_arguments(L):
    E = _lib
    assert bwd(L, C=0) == E.M2RNN_ERR_INVALID_ARG
    assert bwd(L, ckpt=None) == E.M2RNN_ERR_INVALID_ARG
    assert bwd(L, dy=None) == E.M2RNN_ERR_INVALID_ARG
    assert bwd(L, dW=None) == E.M2RNN_ERR_INVALID_ARG
    assert bwd(L, alpha=FAKE) == E.M2RNN_ERR_INVALID_ARG               # sigmoid takes no alpha
    assert bwd(L, gate=E.M2RNN_GATE_EXP_SOFTPLUS) == E.M2RNN_ERR_INVALID_ARG
    assert bwd(L, gate=E.M2RNN_GATE_EXP_SOFTPLUS, alpha=FAKE, beta=FAKE) == E.M2RNN_ERR_INVALID_ARG
    assert bwd(L, V=200) == E.M2RNN_ERR_UNSUPPORTED
    assert bwd(L) == E.M2RNN_ERR_WORKSPACE                             # always needs workspace
    assert bwd(L, ws=FAKE, wsb=64) == E.M2RNN_ERR_WORKSPACE
    big = 1 << 30
    assert bwd(L, ws=FAKE + 4, wsb=big) == E.M2RNN_ERR_INVALID_ARG  # not 16-byte aligned


def test_bwd_noalloc_checks_before_touching_the_device(L):
    # the argument checks of m2rnn_bwd, then the scratch limit, all on the host
    # (no GPU here: a call that got past them would fail with M2RNN_ERR_HIP)
    E = _lib

    def na(**kw):
        a = dict(B=2, T=8, N=1, NQ=None, K=16, V=16, ind=E.M2RNN_F32, sd=E.M2RNN_F32, k=FAKE,
                 v=FAKE, q=FAKE, gate=E.M2RNN_GATE_SIGMOID, logit=FAKE, alpha=None, beta=None,
                 f=FAKE, W=FAKE, w_r=FAKE, H0=None, ckpt=FAKE, C=4, rc=None, dy=FAKE, dHT=None,
                 dk=FAKE, dv=FAKE, dq=FAKE, dlogit=FAKE, dW=FAKE, dw_r=FAKE, dalpha=None,
                 dbeta=None, dH0=None, stream=None)
        a.update(kw)
        if a["NQ"] is None:
            a["NQ"] = a["N"]
        keys = ["B", "T", "N", "NQ", "K", "V", "ind", "sd", "k", "v", "q", "gate", "logit",
                "alpha", "beta", "f", "W", "w_r", "H0", "ckpt", "C", "rc", "dy", "dHT", "dk",
                "dv", "dq", "dlogit", "dW", "dw_r", "dalpha", "dbeta", "dH0", "stream"]
        return L.m2rnn_bwd_noalloc(*[a[k] for k in keys])

    assert na(C=0) == E.M2RNN_ERR_INVALID_ARG
    assert na(dy=None) == E.M2RNN_ERR_INVALID_ARG
    assert na(alpha=FAKE) == E.M2RNN_ERR_INVALID_ARG
    assert na(V=200) == E.M2RNN_ERR_UNSUPPORTED
    big = dict(B=1, T=4096, N=16, K=48, V=128, C=64)
    need = L.m2rnn_workspace_bytes(1, 1, 4096, 16, 16, 48, 128, 64, E.M2RNN_F32)
    assert need > E.NOALLOC_SCRATCH_BYTES
    assert na(**big) == E.M2RNN_ERR_SCRATCH


def step(L, **kw):
    a = dict(B=2, N=2, NQ=None, K=16, V=16, ind=_lib.M2RNN_F32, sd=_lib.M2RNN_F32, k=FAKE,
             v=FAKE, q=FAKE, f=FAKE, W=FAKE, w_r=FAKE, H=FAKE, y=FAKE, stream=None)
    a.update(kw)
    NQ = a["N"] if a["NQ"] is None else a["NQ"]
    return L.m2rnn_step(a["B"], a["N"], NQ, a["K"], a["V"], a["ind"], a["sd"], a["k"], a["v"],
                        a["q"], a["f"], a["W"], a["w_r"], a["H"], a["y"], a["stream"])


def test_step_rejects_bad_arguments(L):
    E = _lib
    assert step(L, B=-1) == E.M2RNN_ERR_INVALID_ARG
    assert step(L, K=0) == E.M2RNN_ERR_INVALID_ARG
    assert step(L, V=0) == E.M2RNN_ERR_INVALID_ARG
    assert step(L, N=4, NQ=3) == E.M2RNN_ERR_INVALID_ARG
    assert step(L, N=4, NQ=0) == E.M2RNN_ERR_INVALID_ARG
    assert step(L, H=None) == E.M2RNN_ERR_INVALID_ARG
    assert step(L, y=None) == E.M2RNN_ERR_INVALID_ARG
    assert step(L, sd=9) == E.M2RNN_ERR_INVALID_ARG
    assert step(L, K=257) == E.M2RNN_ERR_UNSUPPORTED
    assert step(L, V=129) == E.M2RNN_ERR_UNSUPPORTED
    assert step(L, ind=E.M2RNN_F64) == E.M2RNN_ERR_UNSUPPORTED
    # no (b, n) unit: nothing is read or written, nothing launched
    none = dict(k=None, v=None, q=None, f=None, W=None, w_r=None, H=None, y=None)
    assert step(L, B=0, **none) == E.M2RNN_OK
    assert step(L, N=0, NQ=0, **none) == E.M2RNN_OK


def test_block_entry_points_reject_bad_arguments(L):
    E = _lib
    F32, BF, F64 = E.M2RNN_F32, E.M2RNN_BF16, E.M2RNN_F64
    conv = L.m2rnn_conv_silu
    assert conv(-1, 4, 8, BF, F32, FAKE, FAKE, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert conv(2, 4, 0, BF, F32, FAKE, FAKE, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert conv(2, 4, 8, BF, F32, None, FAKE, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert conv(2, 4, 8, BF, BF, FAKE, FAKE, None, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert conv(2, 4, 8, F64, F32, FAKE, FAKE, None, FAKE, None) == E.M2RNN_ERR_UNSUPPORTED
    assert conv(0, 4, 8, BF, F32, None, None, None, None, None) == E.M2RNN_OK
    cb = L.m2rnn_conv_silu_bwd
    # dbias must be given exactly when bias is
    assert cb(2, 4, 8, BF, F32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
              None) == E.M2RNN_ERR_INVALID_ARG
    assert cb(2, 4, 8, BF, F32, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
              None) == E.M2RNN_ERR_INVALID_ARG
    assert cb(2, 4, 8, BF, F32, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, 0,
              None) == E.M2RNN_ERR_WORKSPACE
    assert cb(2, 4, 8, BF, F32, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, 16,
              None) == E.M2RNN_ERR_WORKSPACE
    ws = L.m2rnn_block_workspace_bytes
    # conv: partials [B * ceil(T / 64), C, 5]; norm: per-row 1/rms (64-aligned) and
    # dgamma partials, max(ceil(rows / 256), min(ceil(rows / 4), 1024)) rows of D
    assert ws(0, 2, 130, 8, F32) == ((2 * 3 * 8 * 5 * 4 + 255) // 256) * 256
    assert ws(1, 3, 100, 24, F32) == (((320 + 75 * 24) * 4 + 255) // 256) * 256
    assert ws(1, 3, 100, 24, F64) == (((320 + 75 * 24) * 8 + 255) // 256) * 256
    assert ws(1, 1, 1 << 20, 8, F32) == (((1 << 20) + 4096 * 8) * 4 + 255) // 256 * 256
    assert ws(2, 3, 100, 24, F32) == 0 and ws(0, 0, 100, 24, F32) == 0
    rn = L.m2rnn_gate_rmsnorm
    assert rn(4, 8, BF, F32, -1.0, FAKE, FAKE, FAKE, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert rn(4, 8, BF, F32, float("nan"), FAKE, FAKE, FAKE, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert rn(4, 0, BF, F32, 1e-6, FAKE, FAKE, FAKE, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert rn(4, 8, BF, F32, 1e-6, FAKE, None, FAKE, FAKE, None) == E.M2RNN_ERR_INVALID_ARG
    assert rn(0, 8, BF, F32, 1e-6, None, None, None, None, None) == E.M2RNN_OK
    rb = L.m2rnn_gate_rmsnorm_bwd
    assert rb(4, 8, BF, F32, 1e-6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
              None) == E.M2RNN_ERR_INVALID_ARG
    assert rb(4, 8, BF, F32, 1e-6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
              None) == E.M2RNN_ERR_WORKSPACE


def newton(L, **kw):
    a = dict(B=2, T=8, N=1, NQ=None, K=16, V=16, ind=_lib.M2RNN_F32, k=FAKE, v=FAKE, q=FAKE,
             f=FAKE, W=FAKE, w_r=FAKE, H0=None, iters=3, y=FAKE, HT=None, states=None, res=None,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    NQ = a["N"] if a["NQ"] is None else a["NQ"]
    return L.m2rnn_newton_fwd(a["B"], a["T"], a["N"], NQ, a["K"], a["V"], a["ind"], a["k"],
                              a["v"], a["q"], a["f"], a["W"], a["w_r"], a["H0"], a["iters"],
                              a["y"], a["HT"], a["states"], a["res"], a["ws"], a["wsb"],
                              a["stream"])


def test_newton_workspace_size(L):
    ws = L.m2rnn_newton_workspace_bytes
    # one head, K = V = 16, T = 100: chunks of one step (P = 100), so two
    # iterates X, S, R [100, 16, 16] and E, D [100, 16, 16] and M [100, 16, 16, 16]
    seq = 100 * 16 * 16
    assert ws(1, 100, 1, 16, 16, 0) == (4 * seq + 2 * seq + 16 * seq) * 4
    # the caller's states buffer holds one of the two iterates
    assert ws(1, 100, 1, 16, 16, 1) == (3 * seq + 2 * seq + 16 * seq) * 4
    # enough (unit, row) pairs for a full device: one chunk, no maps
    seq2 = 4 * 32 * 40 * 64 * 16
    assert ws(4, 40, 32, 64, 16, 1) == 3 * seq2 * 4
    assert ws(1, 10, 1, 16, 24, 0) == 0   # V not a multiple of 16
    assert ws(1, 10, 1, 16, 80, 0) == 0   # V above 64
    assert ws(0, 10, 1, 16, 16, 0) == 0   # empty


def test_newton_rejects_bad_arguments(L):
    E = _lib
    assert newton(L, B=-1) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, K=0) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, N=4, NQ=3) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, iters=-1) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, iters=65) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, ind=7) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, y=None) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, f=None) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, H0=FAKE + 4) == E.M2RNN_ERR_INVALID_ARG      # not 16-byte aligned
    assert newton(L, v=FAKE + 8) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, states=FAKE + 8) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, ws=FAKE + 4) == E.M2RNN_ERR_INVALID_ARG
    assert newton(L, ind=E.M2RNN_F64) == E.M2RNN_ERR_UNSUPPORTED
    assert newton(L, V=24) == E.M2RNN_ERR_UNSUPPORTED
    assert newton(L, V=128) == E.M2RNN_ERR_UNSUPPORTED
    assert newton(L, K=257) == E.M2RNN_ERR_UNSUPPORTED
    assert newton(L, ws=None, wsb=0) == E.M2RNN_ERR_WORKSPACE
    assert newton(L, wsb=1000) == E.M2RNN_ERR_WORKSPACE
    # empty: nothing to read; H_T and the residual are NULL here, so nothing is written
    none = dict(k=None, v=None, q=None, f=None, W=None, w_r=None, y=None, ws=None, wsb=0)
    assert newton(L, T=0, **none) == E.M2RNN_OK
    assert newton(L, B=0, **none) == E.M2RNN_OK
