"""ctypes loader for libm2rnn.so (the C ABI declared in include/m2rnn.h).

The library is built in-tree by ``matrix_state_nonlinear_amd.build``.  There is
no fallback: if the shared object is missing or does not load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libm2rnn.so")

M2RNN_OK = 0
M2RNN_ERR_INVALID_ARG = 1
M2RNN_ERR_UNSUPPORTED = 2
M2RNN_ERR_WORKSPACE = 3
M2RNN_ERR_HIP = 4
M2RNN_ERR_SCRATCH = 5
NOALLOC_SCRATCH_BYTES = 64 << 20   # M2RNN_NOALLOC_SCRATCH_BYTES

M2RNN_F32 = 0
M2RNN_BF16 = 1
M2RNN_F64 = 2

M2RNN_GATE_SIGMOID = 0
M2RNN_GATE_EXP_SOFTPLUS = 1

# Every symbol include/m2rnn.h declares, with its ctypes signature.
_i64, _int, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "m2rnn_status_string": (ctypes.c_char_p, [_int]),
    "m2rnn_gates": (_int, [_i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp]),
    "m2rnn_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _int]),
    "m2rnn_fwd": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _int,
                         _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _i64, _vp, _vp, _sz, _vp]),
    "m2rnn_bwd": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _int,
                         _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                         _vp, _sz, _vp]),
    "m2rnn_bwd_noalloc": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _int,
                                 _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp]),
    "m2rnn_step": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int,
                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "m2rnn_newton_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _int]),
    "m2rnn_newton_fwd": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "m2rnn_block_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _int]),
    "m2rnn_conv_silu": (_int, [_i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp]),
    "m2rnn_conv_silu_bwd": (_int, [_i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _sz, _vp]),
    "m2rnn_gate_rmsnorm": (_int, [_i64, _i64, _int, _int, ctypes.c_double, _vp, _vp, _vp, _vp,
                                  _vp]),
    "m2rnn_gate_rmsnorm_bwd": (_int, [_i64, _i64, _int, _int, ctypes.c_double, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
}

_lib = None


class M2RNNError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m matrix_state_nonlinear_amd.build` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().m2rnn_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != M2RNN_OK:
        raise M2RNNError(status, where)
