"""ctypes loader of libsla.so (built in-tree by ``build.py``).

The library is the product: there is no Python or CPU fallback.  Importing
this module raises if the shared object is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libsla.so")

SLA_OK = 0
SLA_ERR_INVALID_ARGUMENT = -1
SLA_ERR_UNSUPPORTED = -2
SLA_ERR_WORKSPACE = -3
SLA_ERR_DEVICE = -4
SLA_ERR_NO_DEVICE = -5

SLA_F32, SLA_BF16 = 0, 1
SLA_STATIC_SCRATCH_BYTES = 64 << 20
(OP_ROUTE, OP_LINEAR_STATES, OP_FORWARD, OP_QUANTIZE_FP8, OP_FORWARD_FP8, OP_ROUTE_TAYLOR,
 OP_FORWARD_PISA, OP_BACKWARD, OP_ROUTE_PISA, OP_RESIDUAL_SUBTRACT) = range(10)


class Problem(ctypes.Structure):
    """Mirror of ``sla_problem`` in include/sla.h."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("k_crit", ctypes.c_int32),
        ("k_marg", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
    ]


_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i32p = ctypes.POINTER(ctypes.c_int32)

SIGNATURES = {
    "sla_validate": (ctypes.c_int, [_P]),
    "sla_num_blocks": (ctypes.c_int, [_P, _i32p, _i32p]),
    "sla_workspace_size": (ctypes.c_int, [_P, ctypes.c_int, ctypes.POINTER(_sz)]),
    "sla_route": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sla_route_quantize": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _sz, _vp]),
    "sla_linear_states_quantize": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "sla_route_noalloc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "sla_route_states": (ctypes.c_int, [_P] + [_vp] * 12 + [_sz, _vp]),
    "sla_validate_lists": (ctypes.c_int, [_P, _vp, _vp, _vp]),
    "sla_route_taylor": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _sz, _vp]),
    "sla_linear_states": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp]),
    "sla_forward": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _sz, _vp]),
    "sla_marginal_sums": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sla_forward_attend": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                          _vp]),
    "sla_quantize_fp8": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp]),
    "sla_forward_fp8": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sla_forward_attend_fp8": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "sla_linear_states_exp": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp]),
    "sla_residual_sums_subtract": (ctypes.c_int, [_P, _vp, _vp, _vp, _sz, _vp]),
    "sla_residual_sums": (ctypes.c_int, [_P, _vp, _vp, _vp, _sz, _vp]),
    "sla_forward_attend_rla": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _sz, _vp]),
    "sla_forward_rla": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _sz, _vp]),
    "sla_pisa_statistics": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sla_forward_attend_pisa": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                               _vp]),
    "sla_route_pisa": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _sz, _vp]),
    "sla_forward_pisa": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sla_backward": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _sz, _vp]),
    "sla_forward_save": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _sz, _vp]),
    "sla_forward_save_fp8": (ctypes.c_int, [_P] + [_vp] * 16 + [_sz, _vp]),
    "sla_backward_saved": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _sz, _vp]),
    "sla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sla_last_error_message": (ctypes.c_char_p, []),
    "sla_version": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int)] * 3),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libsla.so not found at {LIB_PATH}; build it with "
                          "`python block_sparse_linear_route_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
