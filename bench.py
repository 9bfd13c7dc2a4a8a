#!/usr/bin/env python3
"""Benchmark of the sparse-linear attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
route (pool, score, top-k split) -> linear states (H_j, z_j) -> forward
(marginal-state sums, then the fused sparse + linear attention kernel).
Inputs are resident in HBM before timing starts.  Prints one JSON line.

value     executed TFLOP/s of the whole step (executed FLOPs / step time)
roofline  the attention kernel (the dominant one): executed FLOPs per launch
          divided by its mean duration from HIP events on the launch stream,
          against the bf16 dense MFMA peak
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


def load_traffic(workload: str):
    """HBM traffic of the attention kernel from committed PMC summaries, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"attention_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(ATTN_SOURCES):
        return None
    return t.get("hbm_bytes_per_launch")


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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=6,
                    help="heads the oracle runs for the CPU baseline (scaled to all heads)")
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
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (w.q, w.k, w.v))
    alpha = w.alpha.to(dev)
    ws = sla_gpu.forward_workspace(q, kc, km)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        r = sla_gpu.route(q, k, kc, km)
        if ev is not None:
            ev[1].record()
        Hs, zs = sla_gpu.linear_states(k, v)
        if ev is not None:
            ev[2].record()
        sla_gpu.marginal_sums(q, r["marg_idx"], Hs, zs, ws, k_crit=kc)
        if ev is not None:
            ev[3].record()
        o = sla_gpu.forward_attend(q, k, v, r["crit_idx"], alpha, ws, k_marg=km)
        if ev is not None:
            ev[4].record()
        return r, o

    for _ in range(args.warmup):
        r, o = step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        r, o = step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    parts = np.array([[events[i][p].elapsed_time(events[i][p + 1]) for p in range(4)]
                      for i in range(args.steps)])
    route_ms, states_ms, msum_ms, attn_ms = parts.mean(axis=0)
    fwd_ms = msum_ms + attn_ms

    crit = r["crit_idx"].cpu().numpy()
    marg = r["marg_idx"].cpu().numpy()
    f_crit, f_lin, f_sums = executed_flops(crit, marg, N, d)
    f_fwd = f_crit + f_lin + f_sums
    f_step = f_fwd + route_flops(B, H, N, d) + states_flops(B, H, N, d)
    attn_flops = f_crit + f_lin
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    dense_equiv = 4.0 * B * H * N * N * d

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b_ = torch.empty_like(a)
        torch.cuda.synchronize()
        b_.copy_(a)
        torch.cuda.synchronize()

    c = CONFIGS[args.workload]
    out = {
        "metric": METRIC,
        "value": f_step / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: B={B} H={H} N={N} d={d} bf16, block 64, "
                        f"k_crit={kc} k_marg={km} of {(N + 63) // 64} KV blocks"
                        + (f", (t,y,x) grid {c['grid']}" if c.get("grid") else ""),
            "global_batch": B, "seq_len": N, "heads": H, "head_dim": d,
            "k_crit": kc, "k_marg": km, "parallelism": "single GPU",
        },
        "forward_ms": fwd_ms,
        "forward_tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
        "forward_frac_bf16_peak": f_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "breakdown_ms": {"route": route_ms, "linear_states": states_ms,
                         "marginal_sums": msum_ms, "attention": attn_ms},
        "executed_gflop": {"step": f_step / 1e9, "forward": f_fwd / 1e9,
                           "critical_qk_pv": f_crit / 1e9, "linear_apply": f_lin / 1e9,
                           "state_sums": f_sums / 1e9},
        "dense_equivalent": {"gflop": dense_equiv / 1e9,
                             "note": "4 H N^2 d of full attention; its rate at the forward's time",
                             "tflops": dense_equiv / (fwd_ms * 1e-3) / 1e12},
        "roofline": {
            "kernel": "attention_kernel (fused critical online-softmax + linear apply + mix)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": load_traffic(args.workload),
            "flops_per_launch": attn_flops,
            "mean_launch_ms": attn_ms,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, kc, km, f_step, args.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
