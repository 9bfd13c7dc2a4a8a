"""The allocation-free route (sla_route_noalloc, static device scratch)
against sla_route with a caller workspace: identical index lists, class
maps, logits and pooled means, on two calls in a row, the second smaller
than the first (the scratch keeps the first call's contents).  The two take
different selection paths (one fused kernel here; tiled logits through the
workspace, then a selection kernel, in sla_route) whose logits are the same
FMA chains, so the comparison is bit for bit at every row length the fused
kernel has an instance for, ties and all-equal rows included."""
import ctypes

import numpy as np
import pytest
import torch

from block_sparse_linear_route_amd import _lib
from block_sparse_linear_route_amd._lib import lib
from workloads import make_custom, make_workload
from workloads.synth import Workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _s():
    import block_sparse_linear_route_amd as s
    return s


def _noalloc_raw(q, k, kc, km):
    """Direct C-ABI call with preallocated outputs."""
    s = _s()
    B, H, N, d = q.shape
    nb = s.num_blocks(N)
    p = s.make_problem(q, kc, km)
    out = dict(crit_idx=torch.full((B, H, nb, kc), -7, dtype=torch.int32, device=DEV),
               marg_idx=torch.full((B, H, nb, km), -7, dtype=torch.int32, device=DEV),
               block_class=torch.full((B, H, nb, nb), 9, dtype=torch.int8, device=DEV),
               block_logits=torch.full((B, H, nb, nb), float("nan"), device=DEV),
               pooled_q=torch.full((B, H, nb, d), float("nan"), device=DEV),
               pooled_k=torch.full((B, H, nb, d), float("nan"), device=DEV))
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.sla_route_noalloc(ctypes.byref(p), ptr(q), ptr(k), ptr(out["crit_idx"]), ptr(out["marg_idx"]),
                               ptr(out["block_class"]), ptr(out["block_logits"]), ptr(out["pooled_q"]),
                               ptr(out["pooled_k"]), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.SLA_OK, lib.sla_last_error_message()
    return out


def _check_same(w):
    s = _s()
    q, k = w.q.to(DEV), w.k.to(DEV)
    print(f"[noalloc route {w.name} shape {tuple(q.shape)} kc={w.k_crit} km={w.k_marg}]", flush=True)
    got = _noalloc_raw(q, k, w.k_crit, w.k_marg)
    ref = s.route(q, k, w.k_crit, w.k_marg, want_class=True, want_logits=True, want_pooled=True)
    torch.cuda.synchronize()
    for name in ("crit_idx", "marg_idx", "block_class", "block_logits", "pooled_q", "pooled_k"):
        assert torch.equal(got[name], ref[name]), name
    # the binding's wrapper returns the same lists
    via = s.route_noalloc(q, k, w.k_crit, w.k_marg, want_class=True)
    torch.cuda.synchronize()
    assert torch.equal(via["crit_idx"], ref["crit_idx"]) and torch.equal(via["marg_idx"], ref["marg_idx"])
    assert torch.equal(via["block_class"], ref["block_class"])


def test_noalloc_route_equals_route_on_two_calls_second_smaller():
    _check_same(make_workload("video32k"))                                   # 12 heads x 512 blocks
    _check_same(make_custom(1, 2, 1000, 64, dtype="fp32", seed=7, k_crit=3, k_marg=5))


@pytest.mark.parametrize("N, H, kc, km, kind", [
    (64 * 2 - 5, 3, 1, 1, "rand"),        # nkb = 2: 2 keys per lane
    (64 * 128, 2, 13, 26, "rand"),        # nkb = 128
    (64 * 300 + 17, 2, 30, 60, "tie"),    # 8 keys per lane, heavy ties
    (64 * 700, 1, 70, 140, "rand"),       # 16 keys per lane
    (64 * 1500 - 3, 1, 150, 300, "tie"),  # 32 keys per lane
    (64 * 4096, 1, 40, 80, "const"),      # 64 keys per lane, every logit equal
])
def test_noalloc_route_fused_path_equals_split_path(N, H, kc, km, kind):
    if kind == "rand":
        w = make_custom(1, H, N, 128, seed=N % 97, k_crit=kc, k_marg=km)
    else:
        rng = np.random.default_rng(N)
        nkb = (N + 63) // 64
        if kind == "tie":
            pat = rng.standard_normal((4, 128))
            kb = pat[rng.integers(0, 4, nkb)].repeat(64, axis=0)[:N]
        else:
            kb = np.ones((N, 128))
        qv = rng.standard_normal((1, H, N, 128)) if kind == "tie" else np.ones((1, H, N, 128))
        q = torch.tensor(qv, dtype=torch.bfloat16)
        k = torch.tensor(np.broadcast_to(kb, (1, H, N, 128)).copy(), dtype=torch.bfloat16)
        w = Workload(f"{kind}{N}", q, k, k, torch.ones(H), kc, km, {})
    _check_same(w)


def test_noalloc_route_fused_path_equals_split_path_over_two_head_passes():
    # 4096 KV blocks: the keys of one head take 128 MiB, so the split path
    # runs its logits and selection over heads 0-3, then 4-5
    s = _s()
    N, H = 64 * 4096, 6
    assert s.num_blocks(N) == 4096
    w = make_custom(1, H, N, 128, kind="iid", seed=11, k_crit=40, k_marg=80)
    _check_same(w)


def test_noalloc_route_rejects_sizes_past_the_static_scratch():
    s = _s()
    # B * H * nkb = 33 * 1024 > 32768 at head_dim 128: no kernel is launched
    q = torch.zeros(33, 1, 64 * 1024, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(s.SlaError) as e:
        s.route_noalloc(q, q, 4, 8)
    assert e.value.status == _lib.SLA_ERR_WORKSPACE
