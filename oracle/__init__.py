"""Float64 CPU oracle for the TTT-Linear scan (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU path.
"""
from .ttt_oracle import (EPS, LN_EXACT, LN_NONE, LN_ST, inner_grad_vector, input_projections,
                         inner_grad_vector_vjp, layer_norm, ln_jacobian,
                         ln_jacobian_derivative, mlp_inner_grads, rel_max_err, sigmoid, silu,
                         silu_grad, ttt_linear_backward, ttt_linear_forward, ttt_mlp_forward)

__all__ = ["EPS", "LN_EXACT", "LN_NONE", "LN_ST", "inner_grad_vector", "input_projections",
           "inner_grad_vector_vjp", "layer_norm", "ln_jacobian", "ln_jacobian_derivative",
           "mlp_inner_grads", "rel_max_err", "sigmoid", "silu", "silu_grad",
           "ttt_linear_backward", "ttt_linear_forward", "ttt_mlp_forward"]
