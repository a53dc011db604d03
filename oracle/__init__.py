"""fp64 CPU oracle for the M²RNN forward recurrence, its gradients and the layer
front-end that feeds it — test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its binding) never
does, and the two share no code.
"""
from .m2rnn_ref import m2rnn_fwd_ref, round_to_bf16, round_to_f16, widen  # noqa: F401
from .m2rnn_bwd_ref import m2rnn_bwd_ref  # noqa: F401
from .m2rnn_frontend_ref import m2rnn_frontend_ref, sigmoid_ref  # noqa: F401
