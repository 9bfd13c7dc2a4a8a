#!/usr/bin/env python3
"""Benchmark of the sparse-linear attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
route (pool, score, top-k split) -> linear states (H_j, z_j) -> forward
(marginal-state sums, then the fused sparse + linear attention kernel).
Inputs are resident in HBM before timing starts.  Prints one JSON line.

value     executed TFLOP/s of the whole step (executed FLOPs / step time)
roofline  the attention kernel (the dominant one): executed FLOPs per launch
          divided by its mean duration from HIP events on the launch stream,
          against the dense MFMA peak of its dtype (bf16, or fp8 for the
          video32k_fp8 workload, whose step also quantises Q, K and V)
fp8_sparse_branch  (bf16 workloads with d = 128) the same step with the fp8
          sparse branch, timed on the same inputs
cpu_baseline  the fp64 numpy oracle timed on the host cores over a bounded
          sample of the same workload, scaled to the whole step

Executed FLOPs count only work the method performs (no negligible blocks, no
padding), from the index lists the GPU produced:
  forward  sum over (b,h,i): sum_{j in C_i} 4 n_i n_j d      (QK^T and PV)
                           + 2 n_i d (d+1)                    (phi(Q).[S|sigma])
                           + k_m (d^2 + d)                     (state sums)
  route    2 N d (pooling Q and K) + 2 nq nkb d (block logits), per head
  states   sum_j (2 n_j d^2 + n_j d), per head
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-linear attn fwd ms + executed TFLOPS (% MFMA peak) at N=32760, 95% sparse"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
ATTN_SOURCES = ["block_sparse_linear_route_amd/csrc/attention.hip",
                "block_sparse_linear_route_amd/csrc/attention_epilogue.hpp",
                "block_sparse_linear_route_amd/csrc/device_common.hpp"]
ATTN_FP8_SOURCES = ["block_sparse_linear_route_amd/csrc/attention_fp8.hip",
                    "block_sparse_linear_route_amd/csrc/attention_epilogue.hpp",
                    "block_sparse_linear_route_amd/csrc/device_common.hpp"]


def block_sizes(N: int):
    import numpy as np
    nb = (N + 63) // 64
    return np.array([min(64, N - 64 * j) for j in range(nb)], dtype=np.float64)


def executed_flops(crit, marg, N: int, d: int):
    """(critical QK^T+PV, linear apply, state sums) executed FLOPs from index lists."""
    import numpy as np
    n = block_sizes(N)
    nq = len(n)
    n_i = n[None, None, :]
    crit_tokens = n[crit].sum(axis=-1) if crit.shape[-1] else np.zeros(crit.shape[:-1])
    f_crit = float((4.0 * d * n_i * crit_tokens).sum())
    B, H = crit.shape[:2]
    km = marg.shape[-1]
    f_lin = float(2.0 * d * (d + 1) * n.sum() * B * H) if km else 0.0
    f_sums = float(km * (d * d + d) * nq * B * H)
    return f_crit, f_lin, f_sums


def route_flops(B, H, N, d):
    nb = (N + 63) // 64
    return float(B * H * (2 * N * d + 2 * nb * nb * d))


def states_flops(B, H, N, d):
    return float(B * H * (2 * N * d * d + N * d))


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, fp8: bool = False):
    """HBM traffic of the attention kernel from committed PMC summaries, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"attention_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(ATTN_FP8_SOURCES if fp8 else ATTN_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


def load_forward_traffic(workload: str, fp8: bool, B: int, H: int, N: int, d: int):
    """HBM bytes of one forward (marginal sums and the fused kernel) from the
    same committed FETCH_SIZE / WRITE_SIZE summary, against the forward's
    algorithmic bytes: Q, K, V read once (fp8: the E4M3 codes, plus Q in
    bf16 for the linear branch), S_i and sigma_i once, O written once."""
    path = os.path.join(ROOT, "profiles", f"attention_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(ATTN_FP8_SOURCES if fp8 else ATTN_SOURCES):
        return None
    cal = t["copy_calibration"]
    per = t["per_kernel_kib_raw"]
    names = ([n for n in per if n.startswith("marg_prep_kernel<") and n.endswith(", 0>")]
             + [n for n in per if n.startswith("marg_gemm_kernel<") and n.endswith("true, false>")]
             + [t["kernel"]])
    if len(names) != 3 or any(n not in per for n in names):
        return None
    mb = {n: (per[n]["fetch"] * cal["fetch_factor"] + per[n]["write"] * cal["write_factor"]) * 1024
          for n in names}
    nq = (N + 63) // 64
    per_elem = 7 if fp8 else 8          # bytes per (token, feature) of Q, K, V and O
    alg = B * H * (per_elem * N * d + nq * d * d * 2 + nq * d * 4)
    total = sum(mb.values())
    return {"bytes": total, "algorithmic_bytes": float(alg), "ratio": total / alg,
            "per_kernel_mb": {n: v / 1e6 for n, v in mb.items()},
            "note": "per-dispatch FETCH_SIZE + WRITE_SIZE means of the committed profile, each scaled "
                    "by what the counter reads for a plain copy; the marginal sums write S_i and the "
                    "fused kernel reads it back, so S_i crosses HBM twice where the algorithmic count "
                    "has it once, and the mask product reads every state once"}


def make_step(sla_gpu, q, k, v, alpha, kc, km):
    """(step, timed) closures over device-resident inputs.

    step(ev, fp8_step) runs route -> states -> marginal sums -> attention on
    torch's current stream; ev (6 events or None) brackets each op, so each
    event pair times exactly that op's kernels.  timed(n, fp8_step,
    with_events) runs n steps and returns the last routing, the wall ms per
    step and (with events) the mean per-op ms (route, states, -, marginal
    sums, attention)."""
    import numpy as np
    import torch

    ws = sla_gpu.forward_workspace(q, kc, km)
    torch.cuda.synchronize()

    def step(ev=None, fp8_step=False):
        def mark(n):
            if ev is not None:
                ev[n].record()
        mark(0)
        if fp8_step:
            # the pooling pass quantises Q and K, the states pass V
            r = sla_gpu.route_quantize(q, k, kc, km)
            q8, qs, k8, ks = r["q8"], r["q_scale"], r["k8"], r["k_scale"]
        else:
            r = sla_gpu.route(q, k, kc, km)
        mark(1)
        if fp8_step:
            Hs, zs, v8, vs = sla_gpu.linear_states_quantize(k, v)
        else:
            Hs, zs = sla_gpu.linear_states(k, v)
        mark(2)
        mark(3)
        sla_gpu.marginal_sums(q, r["marg_idx"], Hs, zs, ws, k_crit=kc)
        mark(4)
        if fp8_step:
            o = sla_gpu.forward_attend_fp8(q, q8, qs, k8, ks, v8, vs, r["crit_idx"], alpha, ws,
                                           k_marg=km)
        else:
            o = sla_gpu.forward_attend(q, k, v, r["crit_idx"], alpha, ws, k_marg=km)
        mark(5)
        return r, o

    def timed(n_steps, fp8_step, with_events=True):
        events = ([[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_steps)]
                  if with_events else [None] * n_steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_steps):
            r, o = step(events[i], fp8_step)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if not with_events:
            return r, (t1 - t0) * 1e3 / n_steps, None
        parts = np.array([[events[i][p].elapsed_time(events[i][p + 1]) for p in range(5)]
                          for i in range(n_steps)])
        timed.last_parts = parts
        return r, (t1 - t0) * 1e3 / n_steps, parts.mean(axis=0)

    return step, timed


def config_record(sla_gpu, name: str, steps: int, warmup: int, settle_ms: float = 0.0):
    """The step on another named workload: step and forward time, the
    forward's executed TFLOP/s and the attention kernel's fraction of the
    bf16 MFMA peak (same FLOP accounting as the headline line)."""
    import torch
    from workloads import make_workload

    t0 = time.perf_counter()
    w = make_workload(name, cache=False)
    gen_s = time.perf_counter() - t0
    B, H, N, d = w.shape
    kc, km = w.k_crit, w.k_marg
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    alpha = w.alpha.to(dev)
    del w
    step, timed = make_step(sla_gpu, q, k, v, alpha, kc, km)
    settle_steps = 0
    if settle_ms > 0:
        # the GPU idled while the inputs were made: let the clocks ramp again
        torch.cuda.synchronize()
        t_settle = time.perf_counter()
        while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
            step(None, False)
            settle_steps += 1
            torch.cuda.synchronize()
    for _ in range(warmup):
        step(None, False)
    torch.cuda.synchronize()
    r, ms_step, _ = timed(steps, False, with_events=False)
    r, _, parts = timed(steps, False)
    route_ms, states_ms, _, msum_ms, attn_ms = (float(x) for x in parts)
    fwd_ms = msum_ms + attn_ms
    f_crit, f_lin, f_sums = executed_flops(r["crit_idx"].cpu().numpy(),
                                           r["marg_idx"].cpu().numpy(), N, d)
    f_fwd = f_crit + f_lin + f_sums
    f_step = f_fwd + route_flops(B, H, N, d) + states_flops(B, H, N, d)
    attn_tf = (f_crit + f_lin) / (attn_ms * 1e-3) / 1e12
    rec = {
        "workload": f"{name}: B={B} H={H} N={N} d={d} {'fp32' if q.dtype == torch.float32 else 'bf16'}, block 64, "
                    f"k_crit={kc} k_marg={km} of {(N + 63) // 64} KV blocks",
        "steps": steps, "warmup": warmup, "settle_steps": settle_steps,
        "ms_per_step": ms_step,
        "step_tflops": f_step / (ms_step * 1e-3) / 1e12,
        "forward_ms": fwd_ms,
        "forward_tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
        "forward_frac_bf16_peak": f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "breakdown_ms": {"route": route_ms, "linear_states": states_ms,
                         "marginal_sums": msum_ms, "attention": attn_ms},
        "attention_tflops": attn_tf,
        "attention_frac_bf16_peak": attn_tf / PEAK_BF16_TFLOPS,
        "executed_gflop": {"step": f_step / 1e9, "forward": f_fwd / 1e9},
        "input_synthesis_s": gen_s,
    }
    del q, k, v, r
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(w, k_crit, k_marg, f_step, n_heads: int):
    """Oracle timed on whole heads (route, states and forward), scaled to all
    heads of the step."""
    from oracle import sla as ora
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    B, H, N, d = w.shape
    heads = [(b, h) for b in range(B) for h in range(H)][:max(1, n_heads)]
    t0 = time.perf_counter()
    for b, h in heads:
        q64, k64, v64 = (x[b, h].double().numpy() for x in (w.q, w.k, w.v))
        ora.attention_head(q64, k64, v64, float(w.alpha[h]), k_crit, k_marg)
    el = time.perf_counter() - t0
    est = el * (B * H) / len(heads)
    return {
        "value": f_step / est / 1e12,
        "unit": "TFLOP/s",
        "ms_per_step_est": est * 1e3,
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(heads)} of {B * H} heads, each routed, given states and run forward "
                   f"in full by the fp64 oracle ({el:.1f} s); scaled x{B * H / len(heads):.1f} "
                   f"to the whole step"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="video32k")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps run for at least this long before the warm-up steps, so "
                         "that the GPU clocks have ramped up (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=6,
                    help="heads the oracle runs for the CPU baseline (scaled to all heads)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass side measurement")
    ap.add_argument("--no-pisa", action="store_true",
                    help="skip the piecewise exact-or-approximate attention side measurement")
    ap.add_argument("--no-rla", action="store_true",
                    help="skip the residual-linear-attention side measurement")
    ap.add_argument("--other-configs", default="tiny,seq8k,video75k",
                    help="comma-separated bf16 workloads timed after the headline one "
                         "(step, forward, attention fraction of peak); empty for none")
    ap.add_argument("--other-steps", type=int, default=5)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run one device copy of this size (PMC calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_linear_route_amd as sla_gpu
    from workloads import CONFIGS, make_workload

    w = make_workload(args.workload)
    B, H, N, d = w.shape
    kc, km = w.k_crit, w.k_marg
    fp8 = bool(CONFIGS[args.workload].get("fp8"))
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    alpha = w.alpha.to(dev)
    step, timed = make_step(sla_gpu, q, k, v, alpha, kc, km)

    # The clocks ramp up over the first ~100 ms of GPU work: a 20-step window
    # right after 5 warm-up steps measured 0.83 ms per step at video32k where
    # the steady state is 0.75 ms.  Untimed whole steps first, in groups of
    # ten, until at least settle_ms have passed on the device.
    settle_steps = 0
    if args.settle_ms > 0:
        torch.cuda.synchronize()
        t_settle = time.perf_counter()
        while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
            for _ in range(10):
                r, o = step(None, fp8)
            settle_steps += 10
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        r, o = step(None, fp8)
    torch.cuda.synchronize()
    # the timed steps carry no instrumentation; the per-op breakdown comes
    # from a second pass of as many steps with an event between ops
    r, ms_step, _ = timed(args.steps, fp8, with_events=False)
    r, ms_step_instr, parts = timed(args.steps, fp8)
    route_ms, states_ms, _, msum_ms, attn_ms = parts
    route_states_ms = None
    if not fp8:
        # routing and states as one call (sla_route_states: the states pass
        # also pools K), beside the step's two separate calls
        ev_rs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev_rs[0].record()
        for i in range(args.steps):
            sla_gpu.route_states(q, k, v, kc, km)
            ev_rs[i + 1].record()
        torch.cuda.synchronize()
        route_states_ms = float(np.mean([ev_rs[i].elapsed_time(ev_rs[i + 1]) for i in range(args.steps)]))
    fwd_ms = msum_ms + attn_ms
    attn_pct = np.percentile(timed.last_parts[:, 4], [10, 50, 90])

    crit = r["crit_idx"].cpu().numpy()
    marg = r["marg_idx"].cpu().numpy()
    f_crit, f_lin, f_sums = executed_flops(crit, marg, N, d)
    f_fwd = f_crit + f_lin + f_sums
    f_step = f_fwd + route_flops(B, H, N, d) + states_flops(B, H, N, d)
    attn_flops = f_crit + f_lin
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    dense_equiv = 4.0 * B * H * N * N * d
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS

    # the sparse branch alone on the same critical lists (no marginal blocks:
    # the fused kernel skips the linear branch), per-branch context
    ws0 = sla_gpu.forward_workspace(q, kc, 0)
    if fp8:
        codes0 = (r["q8"], r["q_scale"], r["k8"], r["k_scale"],
                  *sla_gpu.linear_states_quantize(k, v)[2:])

        def kern0():
            sla_gpu.forward_attend_fp8(q, *codes0, r["crit_idx"], alpha, ws0, k_marg=0)
    else:
        def kern0():
            sla_gpu.forward_attend(q, k, v, r["crit_idx"], alpha, ws0, k_marg=0)
    kern0()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev0[0].record()
    for i in range(args.steps):
        kern0()
        ev0[i + 1].record()
    torch.cuda.synchronize()
    sparse_only_ms = float(np.mean([ev0[i].elapsed_time(ev0[i + 1]) for i in range(args.steps)]))
    del ws0

    fp8_variant = None
    if not fp8 and d == 128 and w.q.dtype == torch.bfloat16:
        # the fp8 sparse branch on the same inputs (reported beside the bf16 path)
        for _ in range(2):
            step(None, True)
        _, ms8, _ = timed(args.steps, True, with_events=False)
        _, _, parts8 = timed(max(3, args.steps // 2), True)
        r8_ms, st8_ms, _, ms8_sum, ms8_attn = parts8
        fwd8 = ms8_sum + ms8_attn
        fp8_variant = {
            "ms_per_step": ms8,
            "speedup_vs_bf16_step": ms_step / ms8,
            "forward_ms": fwd8,
            "breakdown_ms": {"route_quantize": r8_ms, "linear_states_quantize": st8_ms,
                             "marginal_sums": ms8_sum, "attention_fp8": ms8_attn},
            "quantize_cost_ms": (r8_ms - route_ms) + (st8_ms - states_ms),
            "attention_fp8_tflops": attn_flops / (ms8_attn * 1e-3) / 1e12,
            "attention_fp8_frac_fp8_peak": attn_flops / (ms8_attn * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
            "note": "sla_route_quantize (route plus E4M3 codes of Q and K from the pooling pass), "
                    "sla_linear_states_quantize (states plus codes of V), marginal sums, the fp8 "
                    "attention kernel; same routing, states and executed FLOPs as the bf16 step; "
                    "quantize_cost_ms is the extra time of the two fused passes over the bf16 ones",
        }

    rla_variant = None
    if not fp8 and not args.no_rla:
        # residual linear attention on the same inputs: the critical split of
        # the step, every other block in the residual state
        nb = (N + 63) // 64
        ws_r = sla_gpu.forward_workspace(q, kc, nb - kc)

        def rla_step(ev=None):
            def mark(n):
                if ev is not None:
                    ev[n].record()
            mark(0)
            rr = sla_gpu.route(q, k, kc, nb - kc)
            mark(1)
            He, _ = sla_gpu.linear_states(k, v, feature_map="exp")
            mark(2)
            sla_gpu.residual_sums(q, rr["crit_idx"], He, ws_r)
            mark(3)
            orla = sla_gpu.forward_attend_rla(q, k, v, rr["crit_idx"], alpha, ws_r)
            mark(4)
            return rr, orla

        for _ in range(2):
            rla_step()
        n_r = max(3, args.steps // 2)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_r)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_r):
            rr, _ = rla_step(evs[i])
        torch.cuda.synchronize()
        ms_r = (time.perf_counter() - t0) * 1e3 / n_r
        pr = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)]
                       for i in range(n_r)]).mean(axis=0)
        # the subtraction form of the residual sums (global state minus the
        # critical blocks' states) on the same lists and states
        He_s, _ = sla_gpu.linear_states(k, v, feature_map="exp")
        ws_sub = sla_gpu.residual_workspace_subtract(q, kc)
        sla_gpu.residual_sums_subtract(q, rr["crit_idx"], He_s, ws_sub)
        evr = [torch.cuda.Event(enable_timing=True) for _ in range(n_r + 1)]
        torch.cuda.synchronize()
        evr[0].record()
        for i in range(n_r):
            sla_gpu.residual_sums_subtract(q, rr["crit_idx"], He_s, ws_sub)
            evr[i + 1].record()
        torch.cuda.synchronize()
        sub_ms = float(np.mean([evr[i].elapsed_time(evr[i + 1]) for i in range(n_r)]))
        del He_s, ws_sub
        fr_crit, fr_lin, fr_sums = executed_flops(rr["crit_idx"].cpu().numpy(),
                                                  rr["marg_idx"].cpu().numpy(), N, d)
        fr_fwd = fr_crit + fr_lin + fr_sums
        rla_variant = {
            "ms_per_step": ms_r,
            "forward_ms": float(pr[2] + pr[3]),
            "breakdown_ms": {"route": pr[0], "linear_states_exp": pr[1],
                             "residual_sums": pr[2], "attention_rla": pr[3]},
            "residual_sums_subtraction_form_ms": sub_ms,
            "forward_tflops": fr_fwd / ((pr[2] + pr[3]) * 1e-3) / 1e12,
            "attention_rla_tflops": (fr_crit + fr_lin) / (pr[3] * 1e-3) / 1e12,
            "note": "residual linear attention: same critical split, residual state = the "
                    f"{nb - kc} non-critical blocks, exponential feature map, RMS-normalised "
                    "residual branch; executed FLOPs count the residual sums as k_m (d^2 + d) "
                    "per query block",
        }

    pisa_variant = None
    if not fp8 and not args.no_pisa:
        # piecewise exact-or-approximate attention on the same inputs, routed
        # by the covariance-aware score (its statistics pass also fills the
        # piecewise statistics the fused kernel reads): the critical split
        # exact, every other block by centroid plus the first-order term
        ws_p = sla_gpu.route_pisa(q, k, v, kc, km)["_workspace"]

        def pisa_step(ev=None):
            def mark(n):
                if ev is not None:
                    ev[n].record()
            mark(0)
            rp = sla_gpu.route_pisa(q, k, v, kc, km, workspace=ws_p)
            mark(1)
            op = sla_gpu.forward_attend_pisa(q, k, v, rp["crit_idx"], ws_p)
            mark(2)
            return rp, op

        for _ in range(2):
            pisa_step()
        n_p = max(3, args.steps // 2)
        evp = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_p)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_p):
            rp, _ = pisa_step(evp[i])
        torch.cuda.synchronize()
        ms_p = (time.perf_counter() - t0) * 1e3 / n_p
        pp = np.array([[evp[i][j].elapsed_time(evp[i][j + 1]) for j in range(2)]
                       for i in range(n_p)]).mean(axis=0)
        same_p = ((rp["crit_idx"] == r["crit_idx"]).all(-1)
                  & (rp["marg_idx"] == r["marg_idx"]).all(-1))
        nbk = (N + 63) // 64
        # exact blocks from the covariance-aware lists, one 64-key tile of
        # centroids per 64 KV blocks (only the unselected ones count), the
        # first-order term; the statistics pass as part of the route
        fp_crit, _, _ = executed_flops(rp["crit_idx"].cpu().numpy(), rp["marg_idx"].cpu().numpy(),
                                       N, d)
        fp_zero = 4.0 * B * H * N * d * (nbk - kc)
        fp_corr = 2.0 * B * H * N * d * d
        pisa_variant = {
            "ms_per_step": ms_p,
            "breakdown_ms": {"route_pisa": pp[0], "attention_pisa": pp[1]},
            "attention_pisa_ms": float(pp[1]),
            "attention_pisa_tflops": (fp_crit + fp_zero + fp_corr) / (pp[1] * 1e-3) / 1e12,
            "rows_split_differently_from_mean_score": float(1.0 - same_p.float().mean().item()),
            "note": "sla_route_pisa (pooling, block statistics with the deviations "
                    "M_j = ||H_j - Hbar||_F, covariance-aware top-k) then the fused piecewise "
                    "kernel: critical blocks exact, the other "
                    f"{nbk - kc} blocks per query block through their centroids "
                    f"({(nbk + 63) // 64} pseudo-blocks of 64 centroids in the same online "
                    "softmax), one global first-order correction; FLOPs count 4 n d per "
                    "exact key and per unselected centroid and 2 N d^2 for the correction",
        }

    bwd_variant = None
    if not fp8 and not args.no_backward and w.q.dtype == torch.bfloat16:
        # the backward pass on the same inputs and lists (recomputes the
        # forward, then the gradient kernels), for an upstream gradient dO
        gdo = torch.Generator(device="cpu").manual_seed(4242)
        dout = torch.randn(q.shape, generator=gdo).to(q.dtype).to(dev)
        Hb, zb = sla_gpu.linear_states(k, v)
        kb = sla_gpu.backward(q, k, v, dout, r["crit_idx"], r["marg_idx"], Hb, zb, alpha)
        ws_b = sla_gpu.backward_workspace(q, kc, km)
        n_b = max(3, args.steps // 2)
        evb = [torch.cuda.Event(enable_timing=True) for _ in range(n_b + 1)]
        torch.cuda.synchronize()
        evb[0].record()
        for i_ in range(n_b):
            sla_gpu.backward(q, k, v, dout, r["crit_idx"], r["marg_idx"], Hb, zb, alpha, workspace=ws_b)
            evb[i_ + 1].record()
        torch.cuda.synchronize()
        bwd_ms = float(np.mean([evb[i_].elapsed_time(evb[i_ + 1]) for i_ in range(n_b)]))
        # the same gradients for a training step that runs the forward once:
        # sla_forward_save (the forward, keeping what the backward reads) and
        # sla_backward_saved (the gradient kernels only)
        o_t, _ = sla_gpu.forward_save(q, k, v, r["crit_idx"], r["marg_idx"], Hb, zb, alpha,
                                      workspace=ws_b)
        sla_gpu.backward_saved(q, k, v, dout, r["crit_idx"], r["marg_idx"], alpha, ws_b)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_b)]
        torch.cuda.synchronize()
        for i_ in range(n_b):
            evs[i_][0].record()
            sla_gpu.forward_save(q, k, v, r["crit_idx"], r["marg_idx"], Hb, zb, alpha,
                                 workspace=ws_b, out=o_t)
            evs[i_][1].record()
            sla_gpu.backward_saved(q, k, v, dout, r["crit_idx"], r["marg_idx"], alpha, ws_b)
            evs[i_][2].record()
        torch.cuda.synchronize()
        fsave_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        bsaved_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        # quantisation-aware training step: the fp8 forward keeps its
        # statistics, the bf16 gradient kernels read them
        rq = sla_gpu.route_quantize(q, k, kc, km)
        _, _, v8q, vsq = sla_gpu.linear_states_quantize(k, v)
        codes = (rq["q8"], rq["q_scale"], rq["k8"], rq["k_scale"], v8q, vsq)
        sla_gpu.forward_save_fp8(q, k, v, *codes, r["crit_idx"], r["marg_idx"], Hb, zb, alpha,
                                 workspace=ws_b, out=o_t)
        evq = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_b)]
        torch.cuda.synchronize()
        for i_ in range(n_b):
            evq[i_][0].record()
            sla_gpu.forward_save_fp8(q, k, v, *codes, r["crit_idx"], r["marg_idx"], Hb, zb, alpha,
                                     workspace=ws_b, out=o_t)
            evq[i_][1].record()
            sla_gpu.backward_saved(q, k, v, dout, r["crit_idx"], r["marg_idx"], alpha, ws_b)
            evq[i_][2].record()
        torch.cuda.synchronize()
        fsave8_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evq]))
        bsaved8_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evq]))
        del o_t, rq, codes, v8q, vsq
        # executed FLOPs: the forward again, then per critical (query, key)
        # pair 6 d (dQ kernel: S, dP, dQ) + 8 d (dK/dV kernel: S, dP, dV, dK),
        # 4 d^2 per row on each side of the linear branch, and the marginal
        # gradient sums like the forward's state sums
        f_bwd = f_fwd + 3.5 * f_crit + (8.0 * d * d * N * B * H if km else 0.0) + f_sums
        bwd_variant = {
            "ms": bwd_ms,
            "tflops": f_bwd / (bwd_ms * 1e-3) / 1e12,
            "executed_gflop": f_bwd / 1e9,
            "forward_save_ms": fsave_ms,
            "backward_saved_ms": bsaved_ms,
            "backward_saved_tflops": (f_bwd - f_fwd) / (bsaved_ms * 1e-3) / 1e12,
            "qat_forward_save_fp8_ms": fsave8_ms,
            "qat_backward_saved_ms": bsaved8_ms,
            "qat_note": "quantisation-aware training step: sla_forward_save_fp8 (the fp8 "
                        "sparse branch, keeping its O_s, O_l and normalisers) then "
                        "sla_backward_saved (bf16 gradient kernels); codes made once",
            "saved_note": "training step with the forward run once: sla_forward_save (marginal "
                          "sums and the fused kernel writing O plus O_s, O_l and the normaliser "
                          "into the backward workspace), then sla_backward_saved (gradient "
                          "kernels only; executed FLOPs without the forward's)",
            "note": "sla_backward for fixed lists: marginal sums and the fused forward again "
                    "(writing O_s, O_l and the log2 softmax normaliser), then D_t, sparse dQ, "
                    "linear query side, transposed masks, dH by the mask product, sparse dK/dV, "
                    "linear KV side, dalpha; bf16 inputs, float32 gradients",
        }
        del kb

    # the second-order routing score on the same inputs (route only: the
    # forward that follows is the same kernels on its index lists)
    for _ in range(2):
        sla_gpu.route(q, k, kc, km, score="taylor")
    n_t = max(3, args.steps // 2)
    evt = [torch.cuda.Event(enable_timing=True) for _ in range(n_t + 1)]
    evt[0].record()
    for i in range(n_t):
        rt = sla_gpu.route(q, k, kc, km, score="taylor")
        evt[i + 1].record()
    torch.cuda.synchronize()
    taylor_ms = float(np.mean([evt[i].elapsed_time(evt[i + 1]) for i in range(n_t)]))
    same = ((rt["crit_idx"] == r["crit_idx"]).all(-1) & (rt["marg_idx"] == r["marg_idx"]).all(-1))
    taylor_route = {
        "route_ms": taylor_ms,
        "mean_score_route_ms": float(route_ms),
        "rows_split_differently": float(1.0 - same.float().mean().item()),
        "note": "sla_route_taylor: pooled means plus per-block key variances, score "
                "qbar.kbar/sqrt(d) + log1p(qbar^2 . var / 2d), same top-k split",
    }

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b_ = torch.empty_like(a)
        torch.cuda.synchronize()
        b_.copy_(a)
        torch.cuda.synchronize()

    c = CONFIGS[args.workload]
    traffic = load_traffic(args.workload, fp8)
    out = {
        "metric": METRIC,
        "value": f_step / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step_with_op_events": ms_step_instr,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 sparse branch, bf16/f32 rest" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: B={B} H={H} N={N} d={d} bf16"
                        + (" (E4M3 codes for the sparse branch)" if fp8 else "") + ", block 64, "
                        f"k_crit={kc} k_marg={km} of {(N + 63) // 64} KV blocks"
                        + (f", (t,y,x) grid {c['grid']}" if c.get("grid") else ""),
            "global_batch": B, "seq_len": N, "heads": H, "head_dim": d,
            "k_crit": kc, "k_marg": km, "parallelism": "single GPU",
        },
        "forward_ms": fwd_ms,
        "forward_tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
        "forward_frac_bf16_peak": f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "breakdown_ms": {("route_quantize" if fp8 else "route"): route_ms,
                         ("linear_states_quantize" if fp8 else "linear_states"): states_ms,
                         "marginal_sums": msum_ms, "attention": attn_ms},
        "executed_gflop": {"step": f_step / 1e9, "forward": f_fwd / 1e9,
                           "critical_qk_pv": f_crit / 1e9, "linear_apply": f_lin / 1e9,
                           "state_sums": f_sums / 1e9},
        "dense_equivalent": {"gflop": dense_equiv / 1e9,
                             "note": "4 H N^2 d of full attention; its rate at the forward's time",
                             "tflops": dense_equiv / (fwd_ms * 1e-3) / 1e12},
        "roofline": {
            "kernel": ("attention_fp8_kernel (fp8 critical online-softmax + linear apply + mix)" if fp8
                       else "attention_kernel (fused critical online-softmax + linear apply + mix)"),
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic,
            "flops_per_launch": attn_flops,
            "mean_launch_ms": attn_ms,
            "launch_ms_p10_p50_p90": [float(x) for x in attn_pct],
            "traffic_gbs": None if traffic is None else traffic / (attn_ms * 1e-3) / 1e9,
            "traffic_frac_hbm_peak": None if traffic is None else traffic / (attn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        },
        "route_states_ms": route_states_ms,
        "route_states_note": "sla_route_states (route and states in one call, K read once) "
                             "against breakdown route + linear_states",
        "forward_traffic": load_forward_traffic(args.workload, fp8, B, H, N, d),
        "forward_sparse_only_ms": sparse_only_ms,
        "forward_sparse_only_note": "the fused kernel on the same critical lists with k_marg = 0 "
                                    "(no marginal sums, no linear branch)",
    }
    if fp8:
        out["forward_frac_fp8_peak"] = f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS
    if fp8_variant is not None:
        out["fp8_sparse_branch"] = fp8_variant
    if rla_variant is not None:
        out["residual_linear_attention"] = rla_variant
    if pisa_variant is not None:
        out["piecewise_attention"] = pisa_variant
    out["taylor_routing"] = taylor_route
    if bwd_variant is not None:
        out["backward"] = bwd_variant
    others = [x for x in args.other_configs.split(",") if x and x != args.workload]
    if others:
        out["other_configs"] = {name: config_record(sla_gpu, name, args.other_steps, 2, args.settle_ms)
                                for name in others}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, kc, km, f_step, args.cpu_heads)
        out["cpu_baseline"]["oracle_ms_over_gpu_ms"] = out["cpu_baseline"]["ms_per_step_est"] / ms_step
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
