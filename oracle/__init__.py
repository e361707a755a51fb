"""Plain float64 CPU oracle for the M²RNN recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test-suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP path (no common helpers, tables or constants).

Every function follows the review of "M²RNN: Non-Linear RNNs with Matrix-Valued
States for Scalable Language Modeling" (arXiv:2603.14360v2) and the
pararnn-torch "ParaM2RNN" documentation page; each docstring names the
section / equation it restates.
"""
from .m2rnn_oracle import (  # noqa: F401
    GATE_SIGMOID,
    GATE_EXP_SOFTPLUS,
    softplus,
    sigmoid,
    gates,
    gate_partials,
    forward,
    decode_step,
    backward,
    step_jacobian_dense,
    tangent_growth,
)
from .m2rnn_block import (  # noqa: F401
    silu,
    silu_grad,
    causal_conv,
    conv_silu,
    conv_silu_backward,
    gate_rmsnorm,
    gate_rmsnorm_backward,
)
from .m2rnn_newton import newton_forward, newton_linearize  # noqa: F401
