"""TTT-Linear fast-weight scan for MI355X (gfx950), with the two-layer
(TTT-MLP) inner model as a second scan.

The scans run in hand-written HIP kernels behind the C ABI of
``include/ttt_linear.h`` (``libttt_linear.so``); this package holds the HIP
sources (``csrc/``), their build script, a ctypes binding and the seeded
synthetic input generator.  Importing the package loads nothing; the library
is opened on first use and its absence is an error.
"""
from .binding import (TTT_DUAL, TTT_ERR_ALIAS, TTT_ERR_HIP, TTT_ERR_MODE, TTT_ERR_NULL,
                      TTT_ERR_SHAPE, TTT_ERR_UNSUPPORTED, TTT_ERR_WORKSPACE, TTT_FORCE_VALU,
                      TTT_IN_BF16, TTT_LN_EXACT, TTT_NO_LN, TTT_OK, TTT_SILU_QK,
                      TTT_STATIC_SCRATCH_BYTES, TTTArgumentError, TTTError, backward, check,
                      forward, forward_record, load_library, mlp_forward, mode_bits, project,
                      ttt_linear, ttt_linear_backward, ttt_linear_backward_kernel,
                      ttt_linear_backward_noalloc,
                      ttt_linear_backward_workspace_bytes, ttt_linear_forward,
                      ttt_linear_forward_masked, ttt_linear_forward_record, ttt_linear_kernel,
                      ttt_linear_project, ttt_linear_record_bytes, ttt_linear_validate,
                      ttt_mlp_forward, ttt_mlp_kernel, ttt_mlp_validate, ttt_status_string,
                      ttt_version)

__all__ = ["TTT_DUAL", "TTT_ERR_ALIAS", "TTT_ERR_HIP", "TTT_ERR_MODE", "TTT_ERR_NULL",
           "TTT_ERR_SHAPE", "TTT_ERR_UNSUPPORTED", "TTT_ERR_WORKSPACE", "TTT_FORCE_VALU",
           "TTT_IN_BF16", "TTT_LN_EXACT", "TTT_NO_LN", "TTT_OK", "TTT_SILU_QK",
           "TTT_STATIC_SCRATCH_BYTES", "TTTArgumentError", "TTTError", "backward", "check",
           "forward", "forward_record", "load_library", "mlp_forward", "mode_bits", "project",
           "ttt_linear", "ttt_linear_backward", "ttt_linear_backward_kernel",
           "ttt_linear_backward_noalloc",
           "ttt_linear_backward_workspace_bytes", "ttt_linear_forward",
           "ttt_linear_forward_masked", "ttt_linear_forward_record", "ttt_linear_kernel",
           "ttt_linear_project", "ttt_linear_record_bytes", "ttt_linear_validate",
           "ttt_mlp_forward", "ttt_mlp_kernel", "ttt_mlp_validate", "ttt_status_string",
           "ttt_version"]
