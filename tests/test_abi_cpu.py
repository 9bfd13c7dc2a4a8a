"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/sla.h declares, and validates arguments on the host."""
import ctypes
import os
import re

import pytest

from block_sparse_linear_route_amd import _lib
from block_sparse_linear_route_amd._lib import Problem, lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sla.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 11
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_problem_struct_layout():
    assert ctypes.sizeof(Problem) == 8 * 4 + 3 * 8
    assert Problem.stride_b.offset == 32


def P(**kw):
    base = dict(batch=1, heads=2, seq_len=1000, head_dim=128, block=64, k_crit=2, k_marg=3,
                dtype=_lib.SLA_BF16, stride_b=2 * 1000 * 128, stride_h=1000 * 128, stride_n=128)
    base.update(kw)
    return Problem(**base)


def validate(p):
    return lib.sla_validate(ctypes.byref(p))


@pytest.mark.parametrize("kw,status", [
    ({}, _lib.SLA_OK),
    (dict(head_dim=64, stride_n=64), _lib.SLA_OK),
    (dict(dtype=_lib.SLA_F32), _lib.SLA_OK),
    (dict(head_dim=96), _lib.SLA_ERR_UNSUPPORTED),
    (dict(block=128), _lib.SLA_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.SLA_ERR_UNSUPPORTED),
    (dict(seq_len=64 * 4097), _lib.SLA_ERR_UNSUPPORTED),
    (dict(batch=0), _lib.SLA_ERR_INVALID_ARGUMENT),
    (dict(seq_len=0), _lib.SLA_ERR_INVALID_ARGUMENT),
    (dict(k_crit=0, k_marg=0), _lib.SLA_ERR_INVALID_ARGUMENT),
    (dict(k_crit=10, k_marg=7), _lib.SLA_ERR_INVALID_ARGUMENT),   # 17 > 16 blocks
    (dict(k_crit=16, k_marg=0), _lib.SLA_OK),
    (dict(k_crit=0, k_marg=16), _lib.SLA_OK),
    (dict(k_crit=-1), _lib.SLA_ERR_INVALID_ARGUMENT),
    (dict(stride_n=100), _lib.SLA_ERR_INVALID_ARGUMENT),          # row overlap
    (dict(stride_n=132), _lib.SLA_ERR_INVALID_ARGUMENT),          # 264 B rows: not 16-B multiple
    # packed QKV of 40 heads (row stride 3 * 40 * 128 elements): 139 811
    # tokens span 4 294 963 456 bytes, one more row passes 2^32 - 1
    (dict(seq_len=139811, stride_n=15360, stride_h=128, stride_b=139811 * 15360), _lib.SLA_OK),
    (dict(seq_len=139812, stride_n=15360, stride_h=128, stride_b=139812 * 15360),
     _lib.SLA_ERR_UNSUPPORTED),
    (dict(seq_len=262144, stride_n=15360, stride_h=128, stride_b=0, dtype=_lib.SLA_BF16),
     _lib.SLA_ERR_UNSUPPORTED),
])
def test_validate(kw, status):
    assert validate(P(**kw)) == status
    if status != _lib.SLA_OK:
        assert len(lib.sla_last_error_message()) > 0


def test_validate_null():
    assert lib.sla_validate(None) == _lib.SLA_ERR_INVALID_ARGUMENT


def test_num_blocks_and_workspace():
    p = P(seq_len=32760)
    nq, nkb = ctypes.c_int32(), ctypes.c_int32()
    assert lib.sla_num_blocks(ctypes.byref(p), ctypes.byref(nq), ctypes.byref(nkb)) == 0
    assert nq.value == nkb.value == 512
    n = ctypes.c_size_t()
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_FORWARD, ctypes.byref(n)) == 0
    assert n.value >= 2 * 512 * 128 * 128 * 2 + 2 * 512 * 128 * 4
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_ROUTE, ctypes.byref(n)) == 0
    assert n.value >= 2 * 2 * 512 * 128 * 8
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_ROUTE_TAYLOR, ctypes.byref(n)) == 0
    assert n.value >= 3 * 2 * 512 * 128 * 8
    # PISA: centroids and value means (bf16, 8 tiles of 64 rows), Hbar and partials
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_FORWARD_PISA, ctypes.byref(n)) == 0
    assert n.value >= 2 * (2 * 512 * 128 * 2) + 2 * 128 * 128 * 2 + 2 * 128 * 128 * 4
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_LINEAR_STATES, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.sla_workspace_size(ctypes.byref(p), 99, ctypes.byref(n)) == _lib.SLA_ERR_INVALID_ARGUMENT


def test_status_strings_and_version():
    for s in range(0, -6, -1):
        assert lib.sla_status_string(s)
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.sla_version(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)) == 0
    assert (a.value, b.value, c.value) == (0, 6, 0)


def test_entry_points_reject_bad_arguments_before_any_device_call():
    p = P()
    fake = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x10008)
    st = lib.sla_route(ctypes.byref(p), None, fake, fake, fake, None, None, None, None, fake, 1 << 30, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT
    st = lib.sla_route(ctypes.byref(p), odd, fake, fake, fake, None, None, None, None, fake, 1 << 30, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT
    st = lib.sla_route(ctypes.byref(p), fake, fake, fake, fake, None, None, None, None, fake, 16, None)
    assert st == _lib.SLA_ERR_WORKSPACE
    st = lib.sla_route(ctypes.byref(p), fake, fake, fake, fake, None, None, None, None, None, 0, None)
    assert st == _lib.SLA_ERR_WORKSPACE
    st = lib.sla_route_taylor(ctypes.byref(p), fake, None, fake, fake, None, None, None, None, None,
                              fake, 1 << 30, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT       # k missing
    st = lib.sla_route_taylor(ctypes.byref(p), fake, fake, fake, fake, None, None, None, None,
                              ctypes.c_void_p(0x10002), fake, 1 << 30, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT       # misaligned key_var
    n = ctypes.c_size_t()
    lib.sla_workspace_size(ctypes.byref(p), _lib.OP_ROUTE, ctypes.byref(n))
    st = lib.sla_route_taylor(ctypes.byref(p), fake, fake, fake, fake, None, None, None, None, None,
                              fake, n.value, None)
    assert st == _lib.SLA_ERR_WORKSPACE              # the plain route workspace is too small
    st = lib.sla_linear_states(ctypes.byref(p), fake, None, fake, fake, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT
    # route + states: q, k, v, crit, marg, class, logits, pooled q / k, H, z, ws
    rs = lambda *a: lib.sla_route_states(ctypes.byref(p), *a)
    assert rs(fake, fake, None, fake, fake, None, None, None, None, fake, fake, fake, 1 << 30, None) \
        == _lib.SLA_ERR_INVALID_ARGUMENT             # v missing
    assert rs(fake, fake, fake, fake, fake, None, None, None, None, None, fake, fake, 1 << 30, None) \
        == _lib.SLA_ERR_INVALID_ARGUMENT             # H missing
    assert rs(fake, fake, fake, fake, fake, None, None, None, None, fake, odd, fake, 1 << 30, None) \
        == _lib.SLA_ERR_INVALID_ARGUMENT             # misaligned z
    assert rs(fake, fake, fake, fake, fake, None, None, None, None, fake, fake, fake, 16, None) \
        == _lib.SLA_ERR_WORKSPACE
    st = lib.sla_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, None, fake,
                         None, None, fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT      # alpha missing
    bad = P(head_dim=96)
    st = lib.sla_forward(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_UNSUPPORTED
    st = lib.sla_quantize_fp8(ctypes.byref(p), fake, None, fake, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT
    f32 = P(dtype=_lib.SLA_F32)
    st = lib.sla_forward_fp8(ctypes.byref(f32), *([fake] * 12), None, None, None, fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_UNSUPPORTED
    st = lib.sla_forward_attend_fp8(ctypes.byref(f32), *([fake] * 10), None, None, fake, 1 << 40,
                                    None)
    assert st == _lib.SLA_ERR_UNSUPPORTED            # fp32 Q / O
    d64 = P(head_dim=64, stride_n=64)
    st = lib.sla_forward_attend_fp8(ctypes.byref(d64), *([fake] * 10), None, None, fake, 1 << 40,
                                    None)
    assert st == _lib.SLA_ERR_UNSUPPORTED            # head_dim 64
    st = lib.sla_forward_attend_fp8(ctypes.byref(p), fake, None, *([fake] * 8), None, None,
                                    fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT       # q8 missing
    st = lib.sla_forward_attend_fp8(ctypes.byref(p), *([fake] * 10), None, None, fake, 16, None)
    assert st == _lib.SLA_ERR_WORKSPACE


def test_residual_entry_points_reject_bad_arguments_before_any_device_call():
    fake = ctypes.c_void_p(0x10000)
    p = P()                                  # k_marg = 3 != 16 - 2: not the complement
    st = lib.sla_forward_rla(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, None, None,
                             fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT
    assert b"k_marg must be" in lib.sla_last_error_message()
    r = P(k_crit=2, k_marg=14)               # nkb = 16: every non-critical block
    st = lib.sla_residual_sums(ctypes.byref(r), fake, fake, fake, 16, None)
    assert st == _lib.SLA_ERR_WORKSPACE
    st = lib.sla_residual_sums(ctypes.byref(r), None, fake, fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT      # critical list missing
    st = lib.sla_forward_attend_rla(ctypes.byref(r), fake, fake, fake, fake, None, fake, None, None,
                                    fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT      # alpha missing
    st = lib.sla_linear_states_exp(ctypes.byref(r), fake, None, fake, fake, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT
    all_crit = P(k_crit=16, k_marg=0)        # no residual block: no states needed
    st = lib.sla_residual_sums(ctypes.byref(all_crit), fake, None, fake, 16, None)
    assert st == _lib.SLA_ERR_WORKSPACE


def test_pisa_entry_points_reject_bad_arguments_before_any_device_call():
    fake = ctypes.c_void_p(0x10000)
    p = P()
    st = lib.sla_pisa_statistics(ctypes.byref(p), fake, None, None, fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT       # v missing
    st = lib.sla_pisa_statistics(ctypes.byref(p), fake, fake, ctypes.c_void_p(0x10004), fake,
                                 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT       # misaligned Hbar output
    st = lib.sla_pisa_statistics(ctypes.byref(p), fake, fake, None, fake, 64, None)
    assert st == _lib.SLA_ERR_WORKSPACE
    st = lib.sla_forward_attend_pisa(ctypes.byref(p), fake, fake, fake, None, fake, None, None,
                                     fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT       # k_crit > 0 and no critical list
    st = lib.sla_forward_attend_pisa(ctypes.byref(p), fake, fake, fake, fake, None, None, None,
                                     fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT       # o missing
    n = ctypes.c_size_t()
    lib.sla_workspace_size(ctypes.byref(p), _lib.OP_FORWARD, ctypes.byref(n))
    st = lib.sla_forward_pisa(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, fake,
                              64, None)
    assert st == _lib.SLA_ERR_WORKSPACE
    bad = P(head_dim=96)
    st = lib.sla_forward_pisa(ctypes.byref(bad), fake, fake, fake, fake, fake, None, None, fake,
                              1 << 40, None)
    assert st == _lib.SLA_ERR_UNSUPPORTED


def test_backward_entry_point_rejects_bad_arguments_before_any_device_call():
    fake = ctypes.c_void_p(0x10000)
    p = P()
    st = lib.sla_backward(ctypes.byref(P(dtype=_lib.SLA_F32)), *([fake] * 14), 1 << 40, None)
    assert st == _lib.SLA_ERR_UNSUPPORTED             # float inputs
    st = lib.sla_backward(ctypes.byref(p), fake, fake, fake, None, *([fake] * 9), fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT        # dO missing
    st = lib.sla_backward(ctypes.byref(p), *([fake] * 5), None, *([fake] * 7), fake, 1 << 40, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT        # marginal list missing (k_marg > 0)
    n = ctypes.c_size_t()
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_BACKWARD, ctypes.byref(n)) == 0
    f = ctypes.c_size_t()
    lib.sla_workspace_size(ctypes.byref(p), _lib.OP_FORWARD, ctypes.byref(f))
    assert n.value > f.value + 2 * 2 * 1000 * 128 * 4    # forward workspace + O_s + O_l at least
    st = lib.sla_backward(ctypes.byref(p), *([fake] * 14), f.value, None)
    assert st == _lib.SLA_ERR_WORKSPACE


def test_saved_backward_entry_points_reject_bad_arguments_before_any_device_call():
    fake = ctypes.c_void_p(0x10000)
    p = P()
    n = ctypes.c_size_t()
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_BACKWARD, ctypes.byref(n)) == 0
    # sla_forward_save: q k v crit marg h z alpha o ws
    st = lib.sla_forward_save(ctypes.byref(P(dtype=_lib.SLA_F32)), *([fake] * 10), n.value, None)
    assert st == _lib.SLA_ERR_UNSUPPORTED             # float inputs
    st = lib.sla_forward_save(ctypes.byref(p), *([fake] * 8), None, fake, n.value, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT        # output missing
    st = lib.sla_forward_save(ctypes.byref(p), *([fake] * 5), None, *([fake] * 4), n.value, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT        # states missing (k_marg > 0)
    st = lib.sla_forward_save(ctypes.byref(p), *([fake] * 10), n.value - 1, None)
    assert st == _lib.SLA_ERR_WORKSPACE
    # sla_backward_saved: q k v dout crit marg alpha dq dk dv dalpha ws
    st = lib.sla_backward_saved(ctypes.byref(P(dtype=_lib.SLA_F32)), *([fake] * 12), n.value, None)
    assert st == _lib.SLA_ERR_UNSUPPORTED
    st = lib.sla_backward_saved(ctypes.byref(p), *([fake] * 3), None, *([fake] * 8), n.value, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT        # dO missing
    st = lib.sla_backward_saved(ctypes.byref(p), *([fake] * 10), None, fake, n.value, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT        # dalpha missing
    st = lib.sla_backward_saved(ctypes.byref(p), *([fake] * 12), n.value - 1, None)
    assert st == _lib.SLA_ERR_WORKSPACE


def _device_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_device_visible(), reason="a HIP device is present: fake pointers would reach kernels")
def test_valid_calls_without_a_device_return_no_device():
    # arguments pass validation, then the device check finds no gfx950 GPU
    fake = ctypes.c_void_p(0x10000)
    p = P()
    n = ctypes.c_size_t()
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_ROUTE, ctypes.byref(n)) == 0
    st = lib.sla_route(ctypes.byref(p), fake, fake, fake, fake, None, None, None, None, fake, n.value, None)
    assert st == _lib.SLA_ERR_NO_DEVICE
    assert lib.sla_last_error_message()
    st = lib.sla_linear_states(ctypes.byref(p), fake, fake, fake, fake, None)
    assert st == _lib.SLA_ERR_NO_DEVICE
    st = lib.sla_route_states(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, None, None,
                              fake, fake, fake, n.value, None)
    assert st == _lib.SLA_ERR_NO_DEVICE
    assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_FORWARD, ctypes.byref(n)) == 0
    st = lib.sla_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                         None, None, fake, n.value, None)
    assert st == _lib.SLA_ERR_NO_DEVICE
    st = lib.sla_quantize_fp8(ctypes.byref(p), fake, fake, fake, None)
    assert st == _lib.SLA_ERR_NO_DEVICE


def test_noalloc_route_rejects_sizes_past_the_static_scratch_before_any_device_call():
    fake = ctypes.c_void_p(0x10000)
    assert _lib.SLA_STATIC_SCRATCH_BYTES == 64 << 20
    # route scratch 2 * B*H*nkb*d*8 bytes: 32 * 1024 blocks fit exactly, one more head does not
    fits = P(batch=32, heads=1, seq_len=64 * 1024, stride_h=64 * 1024 * 128, stride_b=64 * 1024 * 128)
    n = ctypes.c_size_t()
    assert lib.sla_workspace_size(ctypes.byref(fits), _lib.OP_ROUTE, ctypes.byref(n)) == 0
    # the caller workspace adds the split selection's keys to the pooled sums
    assert n.value == _lib.SLA_STATIC_SCRATCH_BYTES + 32 * 1024 * 1024 * 8
    big = P(batch=33, heads=1, seq_len=64 * 1024, stride_h=64 * 1024 * 128, stride_b=64 * 1024 * 128)
    st = lib.sla_route_noalloc(ctypes.byref(big), fake, fake, fake, fake, None, None, None, None, None)
    assert st == _lib.SLA_ERR_WORKSPACE
    assert b"static scratch" in lib.sla_last_error_message()
    st = lib.sla_route_noalloc(ctypes.byref(fits), None, fake, fake, fake, None, None, None, None, None)
    assert st == _lib.SLA_ERR_INVALID_ARGUMENT


def test_list_validator_rejects_bad_arguments_before_any_device_call():
    fake = ctypes.c_void_p(0x10000)
    p = P()
    assert lib.sla_validate_lists(ctypes.byref(p), None, fake, None) == _lib.SLA_ERR_INVALID_ARGUMENT
    assert lib.sla_validate_lists(ctypes.byref(p), fake, None, None) == _lib.SLA_ERR_INVALID_ARGUMENT
    assert lib.sla_validate_lists(ctypes.byref(P(head_dim=96)), fake, fake, None) == _lib.SLA_ERR_UNSUPPORTED
    assert lib.sla_validate_lists(None, fake, fake, None) == _lib.SLA_ERR_INVALID_ARGUMENT


@pytest.mark.skipif(_device_visible(), reason="a HIP device is present: fake pointers would reach kernels")
def test_list_validator_without_a_device_returns_no_device():
    fake = ctypes.c_void_p(0x10000)
    assert lib.sla_validate_lists(ctypes.byref(P()), fake, fake, None) == _lib.SLA_ERR_NO_DEVICE
    # a list the count makes unnecessary may be NULL
    assert lib.sla_validate_lists(ctypes.byref(P(k_crit=0)), None, fake, None) == _lib.SLA_ERR_NO_DEVICE


def test_route_workspace_holds_the_keys_of_as_many_heads_as_fit_512_mib():
    # pooled Q and K in float64, then u64 keys [heads][nq][nkb rounded to 64]
    # for min(B*H, 512 MiB / per-head keys) heads (at least one)
    n = ctypes.c_size_t()
    for (b, h, nkb) in [(1, 12, 512), (1, 40, 1182), (2, 4, 4096), (1, 1, 4096), (1, 3, 7)]:
        N = 64 * nkb
        p = P(batch=b, heads=h, seq_len=N, stride_h=N * 128, stride_b=h * N * 128)
        assert lib.sla_workspace_size(ctypes.byref(p), _lib.OP_ROUTE, ctypes.byref(n)) == 0
        align = lambda x: (x + 255) // 256 * 256
        pooled = align(b * h * nkb * 128 * 8)
        nkbp = (nkb + 63) // 64 * 64
        per = nkb * nkbp * 8
        heads = max(1, min(b * h, (512 << 20) // per))
        assert n.value == 2 * pooled + align(heads * per), (b, h, nkb)
