"""M²RNN matrix-state non-linear recurrence on MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI of
``include/m2rnn.h`` (``libm2rnn.so``); this package only marshals torch tensors
(device memory and the current stream) into those calls.  Importing it does not
load the library: the first call does, and fails loudly if it is not built.
"""
from ._lib import (M2RNN_BF16, M2RNN_F32, M2RNN_F64, M2RNN_GATE_EXP_SOFTPLUS,  # noqa: F401
                   M2RNN_GATE_SIGMOID, M2RNNError, LIB_PATH)
from .ops import (m2rnn_conv_silu, m2rnn_conv_silu_bwd, m2rnn_gate_rmsnorm,  # noqa: F401
                  m2rnn_gate_rmsnorm_bwd)
from .ops import (m2rnn_bwd, m2rnn_fwd, m2rnn_gates, m2rnn_step, m2rnn_workspace_bytes,  # noqa: F401
                  m2rnn_status_string)
from .ops import m2rnn_newton_fwd, m2rnn_newton_workspace_bytes  # noqa: F401
from .ops import m2rnn_bwd_noalloc  # noqa: F401
