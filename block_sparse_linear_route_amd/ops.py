"""Torch-facing wrappers of the libsla C ABI (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI;
these functions only allocate outputs and workspaces with torch, pass raw
device pointers and the current HIP stream, and turn status codes into
``SlaError``.  Shapes follow include/sla.h: Q, K, V, O are [B, H, N, d]
with a unit stride on d and equal strides for all four.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import lib

BLOCK = 64


class SlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{lib.sla_status_string(status).decode()} ({status}): {message}")
        self.status = status
        self.message = message


def _check(status: int) -> None:
    if status != _lib.SLA_OK:
        raise SlaError(status, lib.sla_last_error_message().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.SLA_BF16
    if t.dtype == torch.float32:
        return _lib.SLA_F32
    raise SlaError(_lib.SLA_ERR_UNSUPPORTED, f"dtype {t.dtype} (bfloat16 or float32)")


def num_blocks(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


def make_problem(x: torch.Tensor, k_crit: int, k_marg: int) -> _lib.Problem:
    if x.dim() != 4:
        raise SlaError(_lib.SLA_ERR_INVALID_ARGUMENT, "expected a [B, H, N, d] tensor")
    B, H, N, d = x.shape
    sb, sh, sn, sd = x.stride()
    if sd != 1:
        raise SlaError(_lib.SLA_ERR_UNSUPPORTED, "the last dimension must have stride 1")
    return _lib.Problem(B, H, N, d, BLOCK, int(k_crit), int(k_marg), _dtype_code(x), sb, sh, sn)


def _same_layout(ref: torch.Tensor, *others: torch.Tensor):
    """Return tensors sharing ``ref``'s strides (copy the others if needed)."""
    out = []
    for t in others:
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise SlaError(_lib.SLA_ERR_INVALID_ARGUMENT, "Q, K, V must share shape and dtype")
        if t.stride() != ref.stride():
            t = torch.empty_strided(ref.shape, ref.stride(), dtype=ref.dtype, device=ref.device).copy_(t)
        out.append(t)
    return out


def workspace_size(problem: _lib.Problem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.sla_workspace_size(ctypes.byref(problem), op, ctypes.byref(n)))
    return int(n.value)


def _workspace(problem: _lib.Problem, op: int, device) -> Optional[torch.Tensor]:
    n = workspace_size(problem, op)
    if n == 0:
        return None
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + n]


def route(q: torch.Tensor, k: torch.Tensor, k_crit: int, k_marg: int, *, want_class: bool = False,
          want_logits: bool = False, want_pooled: bool = False, score: str = "mean",
          stream=None) -> dict:
    """Pool, score and split: returns crit_idx, marg_idx (+ optional intermediates).

    ``score``: "mean" (the pooled dot product, ``sla_route``) or "taylor"
    (the second-order score with block key variances, ``sla_route_taylor``;
    ``want_pooled`` then also returns ``key_var``)."""
    if score not in ("mean", "taylor"):
        raise SlaError(_lib.SLA_ERR_INVALID_ARGUMENT, f"unknown routing score {score!r}")
    (k,) = _same_layout(q, k)
    p = make_problem(q, k_crit, k_marg)
    B, H, N, d = q.shape
    nb = num_blocks(N)
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(crit_idx=torch.empty((B, H, nb, k_crit), **i32),
               marg_idx=torch.empty((B, H, nb, k_marg), **i32))
    if want_class:
        out["block_class"] = torch.empty((B, H, nb, nb), dtype=torch.int8, device=dev)
    if want_logits:
        out["block_logits"] = torch.empty((B, H, nb, nb), dtype=torch.float32, device=dev)
    if want_pooled:
        out["pooled_q"] = torch.empty((B, H, nb, d), dtype=torch.float32, device=dev)
        out["pooled_k"] = torch.empty((B, H, nb, d), dtype=torch.float32, device=dev)
        if score == "taylor":
            out["key_var"] = torch.empty((B, H, nb, d), dtype=torch.float32, device=dev)
    if score == "taylor":
        ws = _workspace(p, _lib.OP_ROUTE_TAYLOR, dev)
        _check(lib.sla_route_taylor(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(out["crit_idx"]),
                                    _ptr(out["marg_idx"]), _ptr(out.get("block_class")),
                                    _ptr(out.get("block_logits")), _ptr(out.get("pooled_q")),
                                    _ptr(out.get("pooled_k")), _ptr(out.get("key_var")),
                                    _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    else:
        ws = _workspace(p, _lib.OP_ROUTE, dev)
        _check(lib.sla_route(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(out["crit_idx"]),
                             _ptr(out["marg_idx"]), _ptr(out.get("block_class")),
                             _ptr(out.get("block_logits")), _ptr(out.get("pooled_q")),
                             _ptr(out.get("pooled_k")), _ptr(ws), 0 if ws is None else ws.numel(),
                             _stream(stream)))
    out["_workspace"] = ws   # keeps the buffer alive until the caller drops the dict
    return out


def route_pisa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_crit: int, k_marg: int, *,
               want_class: bool = False, want_logits: bool = False, want_pooled: bool = False,
               want_dev: bool = False, workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """``sla_route_pisa``: covariance-aware routing for piecewise attention.
    Returns the route's outputs (``block_dev`` = M_j when ``want_dev``) and
    ``_workspace``, whose leading bytes hold the piecewise statistics that
    ``forward_attend_pisa`` can run from."""
    k, v = _same_layout(q, k, v)
    p = make_problem(q, k_crit, k_marg)
    B, H, N, d = q.shape
    nb = num_blocks(N)
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(crit_idx=torch.empty((B, H, nb, k_crit), **i32),
               marg_idx=torch.empty((B, H, nb, k_marg), **i32))
    if want_class:
        out["block_class"] = torch.empty((B, H, nb, nb), dtype=torch.int8, device=dev)
    if want_logits:
        out["block_logits"] = torch.empty((B, H, nb, nb), dtype=torch.float32, device=dev)
    if want_pooled:
        out["pooled_q"] = torch.empty((B, H, nb, d), dtype=torch.float32, device=dev)
        out["pooled_k"] = torch.empty((B, H, nb, d), dtype=torch.float32, device=dev)
    if want_dev:
        out["block_dev"] = torch.empty((B, H, nb), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else _workspace(p, _lib.OP_ROUTE_PISA, dev)
    _check(lib.sla_route_pisa(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out["crit_idx"]),
                              _ptr(out["marg_idx"]), _ptr(out.get("block_class")),
                              _ptr(out.get("block_logits")), _ptr(out.get("pooled_q")),
                              _ptr(out.get("pooled_k")), _ptr(out.get("block_dev")), _ptr(ws),
                              ws.numel(), _stream(stream)))
    out["_workspace"] = ws
    return out


def validate_lists(q: torch.Tensor, crit_idx: Optional[torch.Tensor],
                   marg_idx: Optional[torch.Tensor], stream=None) -> None:
    """``sla_validate_lists``: raise SlaError if any row's lists hold an index
    outside [0, nkb), a repeat, or a block in both lists (q gives the shape)."""
    kc = int(crit_idx.shape[-1]) if crit_idx is not None else 0
    km = int(marg_idx.shape[-1]) if marg_idx is not None else 0
    p = make_problem(q, kc, km)
    c = crit_idx.contiguous() if crit_idx is not None and kc > 0 else None
    m = marg_idx.contiguous() if marg_idx is not None and km > 0 else None
    _check(lib.sla_validate_lists(ctypes.byref(p), _ptr(c), _ptr(m), _stream(stream)))


def route_noalloc(q: torch.Tensor, k: torch.Tensor, k_crit: int, k_marg: int, *,
                  want_class: bool = False, want_logits: bool = False, want_pooled: bool = False,
                  out: Optional[dict] = None, stream=None) -> dict:
    """``sla_route_noalloc``: the plain route with the library's static device
    scratch in place of a workspace.  ``out`` may hold preallocated outputs
    (crit_idx, marg_idx and the optional ones); missing ones are allocated
    here, so a caller that must not allocate passes all it asks for."""
    (k,) = _same_layout(q, k)
    p = make_problem(q, k_crit, k_marg)
    B, H, N, d = q.shape
    nb = num_blocks(N)
    dev = q.device
    out = dict(out or {})
    shapes = dict(crit_idx=((B, H, nb, k_crit), torch.int32), marg_idx=((B, H, nb, k_marg), torch.int32))
    if want_class:
        shapes["block_class"] = ((B, H, nb, nb), torch.int8)
    if want_logits:
        shapes["block_logits"] = ((B, H, nb, nb), torch.float32)
    if want_pooled:
        shapes["pooled_q"] = ((B, H, nb, d), torch.float32)
        shapes["pooled_k"] = ((B, H, nb, d), torch.float32)
    for name, (shape, dt) in shapes.items():
        if name not in out:
            out[name] = torch.empty(shape, dtype=dt, device=dev)
    _check(lib.sla_route_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(out["crit_idx"]),
                                 _ptr(out["marg_idx"]), _ptr(out.get("block_class")),
                                 _ptr(out.get("block_logits")), _ptr(out.get("pooled_q")),
                                 _ptr(out.get("pooled_k")), _stream(stream)))
    return out


def route_states(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_crit: int, k_marg: int, *,
                 want_class: bool = False, want_logits: bool = False, want_pooled: bool = False,
                 stream=None) -> dict:
    """``route`` and ``linear_states`` in one call (``sla_route_states``): the
    routing outputs plus h_states, z_states; for bf16 inputs K is read once."""
    (k, v) = _same_layout(q, k, v)
    p = make_problem(q, k_crit, k_marg)
    B, H, N, d = q.shape
    nb = num_blocks(N)
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(crit_idx=torch.empty((B, H, nb, k_crit), **i32),
               marg_idx=torch.empty((B, H, nb, k_marg), **i32),
               h_states=torch.empty((B, H, nb, d, d), dtype=torch.bfloat16, device=dev),
               z_states=torch.empty((B, H, nb, d), dtype=torch.float32, device=dev))
    if want_class:
        out["block_class"] = torch.empty((B, H, nb, nb), dtype=torch.int8, device=dev)
    if want_logits:
        out["block_logits"] = torch.empty((B, H, nb, nb), dtype=torch.float32, device=dev)
    if want_pooled:
        out["pooled_q"] = torch.empty((B, H, nb, d), dtype=torch.float32, device=dev)
        out["pooled_k"] = torch.empty((B, H, nb, d), dtype=torch.float32, device=dev)
    ws = _workspace(p, _lib.OP_ROUTE, dev)
    _check(lib.sla_route_states(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out["crit_idx"]),
                                _ptr(out["marg_idx"]), _ptr(out.get("block_class")),
                                _ptr(out.get("block_logits")), _ptr(out.get("pooled_q")),
                                _ptr(out.get("pooled_k")), _ptr(out["h_states"]), _ptr(out["z_states"]),
                                _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return out


def linear_states(k: torch.Tensor, v: torch.Tensor, stream=None, *, feature_map: str = "softmax"):
    """Per-block states: H bf16 [B,H,nkb,d,d], z float32 [B,H,nkb,d].

    ``feature_map``: "softmax" (softmax over the features, the linear branch
    of ``forward``) or "exp" (exp(k) elementwise, the residual branch of
    ``forward_rla``)."""
    if feature_map not in ("softmax", "exp"):
        raise SlaError(_lib.SLA_ERR_INVALID_ARGUMENT, f"unknown feature map {feature_map!r}")
    (v,) = _same_layout(k, v)
    p = make_problem(k, 0, 1)
    B, H, N, d = k.shape
    nb = num_blocks(N)
    Hs = torch.empty((B, H, nb, d, d), dtype=torch.bfloat16, device=k.device)
    zs = torch.empty((B, H, nb, d), dtype=torch.float32, device=k.device)
    fn = lib.sla_linear_states if feature_map == "softmax" else lib.sla_linear_states_exp
    _check(fn(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(Hs), _ptr(zs), _stream(stream)))
    return Hs, zs


def forward(q, k, v, crit_idx, marg_idx, h_states, z_states, alpha, *, branches: bool = False,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Fused sparse + linear forward.  Returns O (and O_s, O_l if ``branches``)."""
    k, v = _same_layout(q, k, v)
    kc, km = int(crit_idx.shape[-1]), int(marg_idx.shape[-1])
    p = make_problem(q, kc, km)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    o_s = o_l = None
    if branches:
        o_s = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o_l = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else _workspace(p, _lib.OP_FORWARD, q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                           _ptr(crit_idx.contiguous()), _ptr(marg_idx.contiguous()),
                           _ptr(h_states), _ptr(z_states), _ptr(alpha), _ptr(out), _ptr(o_s),
                           _ptr(o_l), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return (out, o_s, o_l) if branches else out


def forward_workspace(q: torch.Tensor, k_crit: int, k_marg: int, fp8: bool = False) -> torch.Tensor:
    """A workspace for ``forward`` / ``marginal_sums`` / ``forward_attend``."""
    p = make_problem(q, k_crit, k_marg)
    return _workspace(p, _lib.OP_FORWARD_FP8 if fp8 else _lib.OP_FORWARD, q.device)


def marginal_sums(q, marg_idx, h_states, z_states, workspace, *, k_crit: int, stream=None):
    """First phase of ``forward``: marginal-state sums into ``workspace``."""
    km = int(marg_idx.shape[-1])
    p = make_problem(q, k_crit, km)
    _check(lib.sla_marginal_sums(ctypes.byref(p), _ptr(marg_idx.contiguous()), _ptr(h_states),
                                 _ptr(z_states), _ptr(workspace), workspace.numel(), _stream(stream)))


def forward_attend(q, k, v, crit_idx, alpha, workspace, *, k_marg: int, branches: bool = False,
                   out=None, stream=None):
    """Second phase of ``forward``: fused attention using the sums in ``workspace``."""
    k, v = _same_layout(q, k, v)
    kc = int(crit_idx.shape[-1])
    p = make_problem(q, kc, k_marg)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    o_s = o_l = None
    if branches:
        o_s = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o_l = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_forward_attend(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(crit_idx.contiguous()), _ptr(alpha), _ptr(out), _ptr(o_s),
                                  _ptr(o_l), _ptr(workspace), workspace.numel(), _stream(stream)))
    return (out, o_s, o_l) if branches else out


def residual_sums(q, crit_idx, h_states, workspace, *, stream=None):
    """First phase of ``forward_rla``: S_i = sum of the exponential-map states
    of every non-critical KV block, into ``workspace``."""
    kc = int(crit_idx.shape[-1])
    p = make_problem(q, kc, num_blocks(q.shape[2]) - kc)
    _check(lib.sla_residual_sums(ctypes.byref(p), _ptr(crit_idx.contiguous()), _ptr(h_states),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))


def residual_workspace_subtract(q, k_crit: int):
    """Workspace of ``residual_sums_subtract`` (its leading part is the
    forward workspace ``forward_attend_rla`` reads)."""
    p = make_problem(q, k_crit, num_blocks(q.shape[2]) - k_crit)
    return _workspace(p, _lib.OP_RESIDUAL_SUBTRACT, q.device)


def residual_sums_subtract(q, crit_idx, h_states, workspace, *, stream=None):
    """``residual_sums`` in the subtraction form: the head's global state
    minus the critical blocks' states (workspace from
    ``residual_workspace_subtract``)."""
    kc = int(crit_idx.shape[-1])
    p = make_problem(q, kc, num_blocks(q.shape[2]) - kc)
    _check(lib.sla_residual_sums_subtract(ctypes.byref(p), _ptr(crit_idx.contiguous()),
                                          _ptr(h_states), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))


def forward_attend_rla(q, k, v, crit_idx, alpha, workspace, *, branches: bool = False, out=None,
                       stream=None):
    """Second phase of ``forward_rla``: exact sparse branch, RMS-normalised
    residual branch from the sums in ``workspace``, gated by alpha."""
    k, v = _same_layout(q, k, v)
    kc = int(crit_idx.shape[-1])
    p = make_problem(q, kc, num_blocks(q.shape[2]) - kc)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    o_s = o_l = None
    if branches:
        o_s = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o_l = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_forward_attend_rla(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(crit_idx.contiguous()), _ptr(alpha), _ptr(out),
                                      _ptr(o_s), _ptr(o_l), _ptr(workspace), workspace.numel(),
                                      _stream(stream)))
    return (out, o_s, o_l) if branches else out


def forward_rla(q, k, v, crit_idx, h_states, alpha, *, branches: bool = False, out=None,
                workspace=None, stream=None):
    """Residual linear attention forward: O = alpha O_s + (1 - alpha) RMSNorm(phi(Q) S_i)
    with S_i over every non-critical block (``h_states`` from ``linear_states(...,
    feature_map="exp")``).  Returns O (and O_s, the normalised residual branch if
    ``branches``)."""
    k, v = _same_layout(q, k, v)
    kc = int(crit_idx.shape[-1])
    p = make_problem(q, kc, num_blocks(q.shape[2]) - kc)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    o_s = o_l = None
    if branches:
        o_s = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o_l = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else _workspace(p, _lib.OP_FORWARD, q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_forward_rla(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(crit_idx.contiguous()), _ptr(h_states), _ptr(alpha),
                               _ptr(out), _ptr(o_s), _ptr(o_l), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(stream)))
    return (out, o_s, o_l) if branches else out


def _pisa_problem(x: torch.Tensor, k_crit: int) -> _lib.Problem:
    # the unselected set is every non-critical block: k_marg = nkb - k_crit
    # (the kernels do not read it; it only has to pass validation)
    return make_problem(x, k_crit, num_blocks(x.shape[2]) - k_crit)


def pisa_workspace(q: torch.Tensor) -> torch.Tensor:
    """A workspace for ``pisa_statistics`` / ``forward_attend_pisa`` / ``forward_pisa``."""
    return _workspace(_pisa_problem(q, 0), _lib.OP_FORWARD_PISA, q.device)


def pisa_statistics(k: torch.Tensor, v: torch.Tensor, workspace: torch.Tensor, *,
                    want_hbar: bool = False, stream=None):
    """Block centroids, value means and Hbar into ``workspace``; returns Hbar
    (float32 [B,H,d,d], value-major: [c][a] = Hbar[a][c]) if ``want_hbar``."""
    (v,) = _same_layout(k, v)
    p = _pisa_problem(k, 0)
    B, H, N, d = k.shape
    hb = torch.empty((B, H, d, d), dtype=torch.float32, device=k.device) if want_hbar else None
    _check(lib.sla_pisa_statistics(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(hb), _ptr(workspace),
                                   workspace.numel(), _stream(stream)))
    return hb


def forward_attend_pisa(q, k, v, crit_idx, workspace, *, branches: bool = False, out=None,
                        stream=None):
    """The fused pass of ``forward_pisa`` from a workspace ``pisa_statistics`` filled."""
    k, v = _same_layout(q, k, v)
    p = _pisa_problem(q, int(crit_idx.shape[-1]))
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    o_s = o_c = None
    if branches:
        o_s = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o_c = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check(lib.sla_forward_attend_pisa(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(crit_idx.contiguous()), _ptr(out), _ptr(o_s), _ptr(o_c),
                                       _ptr(workspace), workspace.numel(), _stream(stream)))
    return (out, o_s, o_c) if branches else out


def forward_pisa(q, k, v, crit_idx, *, branches: bool = False, out=None, workspace=None,
                 stream=None):
    """Piecewise exact-or-approximate attention: the critical blocks exactly,
    every other block through its centroid (zero order) plus one global
    first-order correction, all in one softmax.  Returns O (and the softmax
    part and the correction part, O = their sum, if ``branches``)."""
    k, v = _same_layout(q, k, v)
    p = _pisa_problem(q, int(crit_idx.shape[-1]))
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    o_s = o_c = None
    if branches:
        o_s = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o_c = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else _workspace(p, _lib.OP_FORWARD_PISA, q.device)
    _check(lib.sla_forward_pisa(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(crit_idx.contiguous()), _ptr(out), _ptr(o_s), _ptr(o_c),
                                _ptr(ws), ws.numel(), _stream(stream)))
    return (out, o_s, o_c) if branches else out


def backward_workspace(q: torch.Tensor, k_crit: int, k_marg: int) -> torch.Tensor:
    """A workspace for ``backward``."""
    return _workspace(make_problem(q, k_crit, k_marg), _lib.OP_BACKWARD, q.device)


def backward(q, k, v, dout, crit_idx, marg_idx, h_states, z_states, alpha, *, workspace=None,
             stream=None):
    """Gradients of ``forward`` for fixed block lists: (dq, dk, dv) float32
    [B,H,N,d] and dalpha float32 [H].  bf16 inputs only."""
    k, v, dout = _same_layout(q, k, v, dout)
    kc, km = int(crit_idx.shape[-1]), int(marg_idx.shape[-1])
    p = make_problem(q, kc, km)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(q.shape, **f32)
    dv = torch.empty(q.shape, **f32)
    da = torch.empty(q.shape[1], **f32)
    ws = workspace if workspace is not None else _workspace(p, _lib.OP_BACKWARD, q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                            _ptr(crit_idx.contiguous()), _ptr(marg_idx.contiguous()),
                            _ptr(h_states), _ptr(z_states), _ptr(alpha), _ptr(dq), _ptr(dk),
                            _ptr(dv), _ptr(da), _ptr(ws), ws.numel(), _stream(stream)))
    return dq, dk, dv, da


def forward_save(q, k, v, crit_idx, marg_idx, h_states, z_states, alpha, *, workspace=None,
                 out=None, stream=None):
    """``forward`` for a training step: returns (O, workspace), the workspace
    (of ``backward_workspace`` size) holding what ``backward_saved`` reads
    instead of recomputing the forward.  bf16 inputs only."""
    k, v = _same_layout(q, k, v)
    kc, km = int(crit_idx.shape[-1]), int(marg_idx.shape[-1])
    p = make_problem(q, kc, km)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    ws = workspace if workspace is not None else _workspace(p, _lib.OP_BACKWARD, q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_forward_save(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(crit_idx.contiguous()), _ptr(marg_idx.contiguous()),
                                _ptr(h_states), _ptr(z_states), _ptr(alpha), _ptr(out), _ptr(ws),
                                ws.numel(), _stream(stream)))
    return out, ws


def forward_save_fp8(q, k, v, q8, q_scale, k8, k_scale, v8, v_scale, crit_idx, marg_idx, h_states,
                     z_states, alpha, *, workspace=None, out=None, stream=None):
    """The fp8 forward for quantisation-aware training: returns (O, workspace),
    the workspace holding the fp8 forward's O_s, O_l and normalisers for
    ``backward_saved`` (bf16 gradients, the quantisation passed through)."""
    k, v = _same_layout(q, k, v)
    kc, km = int(crit_idx.shape[-1]), int(marg_idx.shape[-1])
    p = make_problem(q, kc, km)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    ws = workspace if workspace is not None else _workspace(p, _lib.OP_BACKWARD, q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    codes = [t.contiguous() for t in (q8, q_scale, k8, k_scale, v8, v_scale)]
    _check(lib.sla_forward_save_fp8(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                    *[_ptr(t) for t in codes],
                                    _ptr(crit_idx.contiguous()), _ptr(marg_idx.contiguous()),
                                    _ptr(h_states), _ptr(z_states), _ptr(alpha), _ptr(out),
                                    _ptr(ws), ws.numel(), _stream(stream)))
    return out, ws


def backward_saved(q, k, v, dout, crit_idx, marg_idx, alpha, workspace, *, stream=None):
    """``backward`` without its forward part: ``workspace`` is the one
    ``forward_save`` filled for the same inputs, lists and alpha."""
    k, v, dout = _same_layout(q, k, v, dout)
    kc, km = int(crit_idx.shape[-1]), int(marg_idx.shape[-1])
    p = make_problem(q, kc, km)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(q.shape, **f32)
    dv = torch.empty(q.shape, **f32)
    da = torch.empty(q.shape[1], **f32)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_backward_saved(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                  _ptr(crit_idx.contiguous()), _ptr(marg_idx.contiguous()),
                                  _ptr(alpha), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv, da


def route_quantize(q: torch.Tensor, k: torch.Tensor, k_crit: int, k_marg: int, *,
                   want_class: bool = False, stream=None) -> dict:
    """``sla_route_quantize``: ``route`` (mean score) plus the E4M3 codes and
    scales of Q and K from the pooling pass: ``q8``, ``q_scale``, ``k8``, ``k_scale``."""
    (k,) = _same_layout(q, k)
    p = make_problem(q, k_crit, k_marg)
    B, H, N, d = q.shape
    nb = num_blocks(N)
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(crit_idx=torch.empty((B, H, nb, k_crit), **i32),
               marg_idx=torch.empty((B, H, nb, k_marg), **i32),
               q8=torch.empty((B, H, N, d), dtype=torch.uint8, device=dev),
               q_scale=torch.empty((B, H, nb), dtype=torch.float32, device=dev),
               k8=torch.empty((B, H, N, d), dtype=torch.uint8, device=dev),
               k_scale=torch.empty((B, H, nb), dtype=torch.float32, device=dev))
    if want_class:
        out["block_class"] = torch.empty((B, H, nb, nb), dtype=torch.int8, device=dev)
    ws = _workspace(p, _lib.OP_ROUTE, dev)
    _check(lib.sla_route_quantize(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(out["crit_idx"]),
                                  _ptr(out["marg_idx"]), _ptr(out.get("block_class")), None, None,
                                  None, _ptr(out["q8"]), _ptr(out["q_scale"]), _ptr(out["k8"]),
                                  _ptr(out["k_scale"]), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream)))
    out["_workspace"] = ws
    return out


def linear_states_quantize(k: torch.Tensor, v: torch.Tensor, stream=None):
    """``sla_linear_states_quantize``: (H, z) of ``linear_states`` plus the
    E4M3 codes (uint8 [B,H,N,d]) and scales (float32 [B,H,nb]) of V."""
    (v,) = _same_layout(k, v)
    p = make_problem(k, 0, 1)
    B, H, N, d = k.shape
    nb = num_blocks(N)
    Hs = torch.empty((B, H, nb, d, d), dtype=torch.bfloat16, device=k.device)
    zs = torch.empty((B, H, nb, d), dtype=torch.float32, device=k.device)
    v8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=k.device)
    vs = torch.empty((B, H, nb), dtype=torch.float32, device=k.device)
    _check(lib.sla_linear_states_quantize(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(Hs), _ptr(zs),
                                          _ptr(v8), _ptr(vs), _stream(stream)))
    return Hs, zs, v8, vs


def quantize_fp8(x: torch.Tensor, stream=None):
    """Per-block E4M3 codes (uint8 [B,H,N,d]) and float32 scales [B,H,nb]."""
    p = make_problem(x, 0, 1)
    B, H, N, d = x.shape
    codes = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, num_blocks(N)), dtype=torch.float32, device=x.device)
    _check(lib.sla_quantize_fp8(ctypes.byref(p), _ptr(x), _ptr(codes), _ptr(scales),
                                _stream(stream)))
    return codes, scales


def forward_fp8(q, q8, q_s, k8, k_s, v8, v_s, crit_idx, marg_idx, h_states, z_states, alpha, *,
                branches: bool = False, out=None, workspace=None, stream=None):
    """Forward with the fp8 sparse branch (codes and scales from ``quantize_fp8``)."""
    kc, km = int(crit_idx.shape[-1]), int(marg_idx.shape[-1])
    p = make_problem(q, kc, km)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    o_s = o_l = None
    if branches:
        o_s = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o_l = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else _workspace(p, _lib.OP_FORWARD_FP8, q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_forward_fp8(ctypes.byref(p), _ptr(q), _ptr(q8), _ptr(q_s), _ptr(k8), _ptr(k_s),
                               _ptr(v8), _ptr(v_s), _ptr(crit_idx.contiguous()),
                               _ptr(marg_idx.contiguous()), _ptr(h_states), _ptr(z_states),
                               _ptr(alpha), _ptr(out), _ptr(o_s), _ptr(o_l), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(stream)))
    return (out, o_s, o_l) if branches else out


def forward_attend_fp8(q, q8, q_s, k8, k_s, v8, v_s, crit_idx, alpha, workspace, *, k_marg: int,
                       branches: bool = False, out=None, stream=None):
    """Second phase of ``forward_fp8``: the fused fp8-sparse / linear attention
    reading the marginal sums ``marginal_sums`` left in ``workspace``."""
    kc = int(crit_idx.shape[-1])
    p = make_problem(q, kc, k_marg)
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    o_s = o_l = None
    if branches:
        o_s = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        o_l = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    alpha = alpha.to(device=q.device, dtype=torch.float32).contiguous()
    _check(lib.sla_forward_attend_fp8(ctypes.byref(p), _ptr(q), _ptr(q8), _ptr(q_s), _ptr(k8),
                                      _ptr(k_s), _ptr(v8), _ptr(v_s), _ptr(crit_idx.contiguous()),
                                      _ptr(alpha), _ptr(out), _ptr(o_s), _ptr(o_l),
                                      _ptr(workspace), workspace.numel(), _stream(stream)))
    return (out, o_s, o_l) if branches else out


def sla_attention(q, k, v, alpha, k_crit: int, k_marg: int, *, fp8: bool = False, stream=None):
    """Route + linear states + forward in one call (returns O)."""
    r = route(q, k, k_crit, k_marg, stream=stream)
    Hs, zs = linear_states(k, v, stream=stream)
    if fp8:
        q8, qs = quantize_fp8(q, stream=stream)
        k8, ks = quantize_fp8(k, stream=stream)
        v8, vs = quantize_fp8(v, stream=stream)
        return forward_fp8(q, q8, qs, k8, ks, v8, vs, r["crit_idx"], r["marg_idx"], Hs, zs, alpha,
                           stream=stream)
    return forward(q, k, v, r["crit_idx"], r["marg_idx"], Hs, zs, alpha, stream=stream)


def version():
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib.sla_version(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value
