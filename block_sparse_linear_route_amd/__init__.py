"""Sparse-linear attention forward for MI355X (gfx950).

The computation lives in ``lib/libsla.so`` (hand-written HIP kernels behind
the C ABI declared in ``include/sla.h``); this package is its thin Python
binding.  Importing it fails if the library has not been built.
"""
from .ops import (  # noqa: F401
    SlaError,
    backward,
    backward_saved,
    backward_workspace,
    forward,
    forward_attend,
    forward_attend_fp8,
    forward_attend_pisa,
    forward_attend_rla,
    forward_fp8,
    forward_pisa,
    forward_rla,
    forward_save,
    forward_save_fp8,
    forward_workspace,
    linear_states,
    linear_states_quantize,
    make_problem,
    marginal_sums,
    num_blocks,
    pisa_statistics,
    pisa_workspace,
    quantize_fp8,
    residual_sums,
    residual_sums_subtract,
    residual_workspace_subtract,
    route,
    route_noalloc,
    route_states,
    validate_lists,
    route_pisa,
    route_quantize,
    sla_attention,
    version,
    workspace_size,
)
